/*
 * libgdn.h -- C ABI of libgdn, hand-written HIP kernels (AMD Instinct MI355X,
 * gfx950) for the gated-delta-rule (GDN) linear-attention mixer of the
 * Qwen3.5 hybrid models.
 *
 * The mixer, per layer and per stream: a depthwise causal conv1d of width 4
 * over the packed q/k/v channels, whose last three raw input rows are the
 * stream's conv tail; SiLU on every channel; q and k L2-normalised per key
 * head (q also scaled by dk^-1/2); then, per value head, the gated delta rule
 * (Yang, Kautz and Hatamizadeh, "Gated Delta Networks", 2024)
 *     S <- alpha S (I - beta k k^T) + beta v k^T,     o = S q,
 *     alpha = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b).
 * The engine on the pages keeps this glue (gated delta rule and causal
 * convolution) in qwen35.cu: page "perf(qwen3_5 cuda): deliver the first
 * token before drafting", commit note on the MLX affine 4-bit checkpoint.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller; libgdn never
 *    allocates, frees or keeps them, and keeps no state between calls.
 *    bf16 values travel as their 16-bit patterns (uint16_t).
 *  - Channels of a packed row: C = 2*hk*dk + hv*dv, ordered [q | k | v], each
 *    head-major.  Value head h reads key head h / (hv / hk).
 *  - The recurrent state of a stream is fp32 [hv][dk][dv] with dv contiguous:
 *    it stores S^T, so element [h][i][j] is S_h[j][i].
 *  - The conv tail of a stream is bf16 [3][C]: the last three raw (pre-conv)
 *    rows, oldest first.  Conv weights are fp32 [C][4]; tap 3 multiplies the
 *    current row, tap j the row 3 - j before it.  There is no conv bias.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  All host-visible arguments are checked before anything is
 *    launched: a refused call returns a negative status and touches no
 *    output.  gdn_last_error() then describes the refusal (per thread).
 *  - Arguments that live on the device (row starts, parents, accepted rows)
 *    cannot be checked without a synchronisation.  Their rules are stated
 *    per call; a stream whose device-side layout breaks them is skipped by
 *    the kernels (its outputs are left untouched).  gdn_check_layout() checks
 *    host copies of them.
 *  - Supported geometry: dk in {64, 128}; dv in {64, 128}; hv % hk == 0;
 *    conv_width == 4.  Windows hold at most 16 rows.
 */
#ifndef LIBGDN_H
#define LIBGDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_MAX_WINDOW_ROWS 16

typedef struct gdn_shape {
    int32_t hk;          /* key heads                        */
    int32_t hv;          /* value heads, a multiple of hk    */
    int32_t dk;          /* key (and query) head size        */
    int32_t dv;          /* value head size                  */
    int32_t conv_width;  /* must be 4                        */
} gdn_shape;

typedef struct gdn_params {
    const float *conv_w;   /* [C][4] fp32, device */
    const float *a_log;    /* [hv]   fp32, device */
    const float *dt_bias;  /* [hv]   fp32, device */
} gdn_params;

enum gdn_status {
    GDN_OK = 0,
    GDN_EINVAL = -1,        /* malformed argument (null pointer, bad size) */
    GDN_EUNSUPPORTED = -2,  /* well-formed but outside the supported shapes */
    GDN_EWORKSPACE = -3,    /* workspace missing or too small               */
    GDN_EHIP = -4           /* the HIP runtime refused a launch             */
};

/* Name of a status code ("GDN_OK", "GDN_EINVAL", ...); never NULL. */
const char *gdn_status_name(int status);

/* Text of the last refusal on the calling thread ("" if none). */
const char *gdn_last_error(void);

/* Number of conv channels C of a shape, or -1 if the shape is refused. */
int32_t gdn_channels(const gdn_shape *shape);

/*
 * One-row decode step for n_streams streams, updating state and tail in
 * place (one-row steps and prompt passes update a stream's state in place:
 * page "perf(qwen3_5 cuda): deliver the first token before drafting", commit
 * note on tree-shaped verify windows).
 *   qkv       [n][C] bf16      row of each stream
 *   a, b      [n][hv] bf16     gate inputs
 *   conv_tail [n][3][C] bf16   in/out
 *   state     [n][hv][dk][dv]  fp32 in/out
 *   out       [n][hv][dv] fp32 o of each value head
 * The result equals, bit for bit, a one-row gdn_recur_window followed by
 * gdn_commit of that row.  Extra limit: (hv/hk) * dv <= 512.
 */
int gdn_conv_step(const gdn_shape *shape, const gdn_params *params, int32_t n_streams,
                  const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                  uint16_t *conv_tail, float *state, float *out, void *stream);

/*
 * Verify windows of several streams in one pass, recording every row's state
 * and conv tail.  Windows hold up to 16 rows, every stream's window is packed
 * back to back (up to 16 streams of 16 rows were taken together on the page
 * "perf(qwen27 cuda): reduce repeated-prompt TTFT", commit note on the
 * qwen3_5 checkpoint with the 27B's shapes), and each row's recurrence and
 * conv tail are recorded so that any prefix can be kept (page "perf(qwen3_5
 * cuda): deliver the first token before drafting", commit note on the MLX
 * affine 4-bit checkpoint).  Row t of stream s is packed row row_start[s]+t
 * and follows row t-1 (row 0 follows the stream's state and tail).
 *   row_start  [n+1] int32, device: 0 <= row_start[s] <= row_start[s+1]
 *              <= total_rows and row_start[s+1] - row_start[s] <= max_rows
 *   max_rows   1..16, a bound on every window's length
 *   qkv        [total_rows][C] bf16;  a, b [total_rows][hv] bf16
 *   conv_tail  [n][3][C] bf16, state [n][hv][dk][dv] fp32: read only
 *   out        [total_rows][hv][dv] fp32
 *   tail_snap  [total_rows][3][C] bf16: the tail after each row
 *   state_snap [total_rows][hv][dk][dv] fp32: the state after each row
 * Each row's results equal, bit for bit, gdn_conv_step applied row by row,
 * whatever the other streams in the pass and whatever the packing offset.
 */
int gdn_recur_window(const gdn_shape *shape, const gdn_params *params, int32_t n_streams,
                     int32_t total_rows, int32_t max_rows, const int32_t *row_start,
                     const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                     const uint16_t *conv_tail, const float *state, float *out,
                     uint16_t *tail_snap, float *state_snap, void *stream);

/*
 * Tree-shaped verify windows: each row names its parent, and the conv taps
 * and the delta rule follow that row's own branch (page "perf(qwen3_5 cuda):
 * deliver the first token before drafting", commit note on tree-shaped verify
 * windows).  Same arguments as gdn_recur_window, plus
 *   parent [total_rows] int32, device: the parent's local index within its
 *          stream's window, -1 for a row that follows the stream's own state
 *          and tail; -1 <= parent[row_start[s]+t] < t.
 * A row's state starts from its parent's recorded state, and its conv taps are
 * its three nearest ancestors' raw rows, continuing into the stream's tail.
 * Every root-to-row path equals, bit for bit, gdn_recur_window over that path.
 */
int gdn_recur_tree(const gdn_shape *shape, const gdn_params *params, int32_t n_streams,
                   int32_t total_rows, int32_t max_rows, const int32_t *row_start,
                   const int32_t *parent, const uint16_t *qkv, const uint16_t *a,
                   const uint16_t *b, const uint16_t *conv_tail, const float *state,
                   float *out, uint16_t *tail_snap, float *state_snap, void *stream);

/*
 * Commit of the accepted rows: only each stream's accepted path is kept (page
 * "perf(qwen27 cuda): reduce repeated-prompt TTFT", commit note on the qwen3_5
 * checkpoint with the 27B's shapes).  Copies the accepted row's recorded state
 * and tail over the stream's state and conv_tail.
 *   row_start  [n+1] int32, device: the layout of the gdn_recur_window /
 *              gdn_recur_tree call that recorded the snapshots
 *   accept_row [n] int32, device: the packed index of the stream's accepted
 *              row, within its own window [row_start[s], row_start[s+1]), or
 *              -1 to keep the stream as it is.  Any other value, or a window
 *              that ends past total_rows, skips the stream (a row of another
 *              stream's window is never copied).
 *   tail_snap [total_rows][3][C], state_snap [total_rows][hv][dk][dv]: read
 */
int gdn_commit(const gdn_shape *shape, int32_t n_streams, int32_t total_rows,
               const int32_t *row_start, const int32_t *accept_row, const uint16_t *tail_snap,
               const float *state_snap, uint16_t *conv_tail, float *state, void *stream);

/*
 * Verify windows or trees that LOG every row instead of recording its state
 * and tail: a verify logs its rows' decay, write and key, and keeping a row
 * replays the kept path onto the recurrence (page "perf(qwen3_5 cuda):
 * deliver the first token before drafting", commit note on tree-shaped verify
 * windows).  Same arguments as gdn_recur_tree, with parent == NULL for chain
 * windows, and in place of tail_snap / state_snap:
 *   log_alpha [total_rows][hv] fp32      alpha of each (row, value head)
 *   log_delta [total_rows][hv][dv] fp32  the row's write delta, with
 *             M_row = alpha M_parent + khat delta^T in the stored form M = S^T
 *             (delta = beta (v - alpha M_parent^T khat))
 *   log_key   [total_rows][hk][dk] fp32  khat of each (row, key head)
 * out equals, bit for bit, what gdn_recur_window / gdn_recur_tree write; the
 * log is about 1/100 of the recorded states' bytes at dk = dv = 128, and no
 * per-row state is ever written.
 */
int gdn_recur_log(const gdn_shape *shape, const gdn_params *params, int32_t n_streams,
                  int32_t total_rows, int32_t max_rows, const int32_t *row_start,
                  const int32_t *parent, const uint16_t *qkv, const uint16_t *a,
                  const uint16_t *b, const uint16_t *conv_tail, const float *state, float *out,
                  float *log_alpha, float *log_delta, float *log_key, void *stream);

/*
 * Commit by replay after gdn_recur_log (same page and note: keeping a row
 * replays its path in one pass and carries the path's own entries into
 * place).
 * accept_row [n] int32, device: the packed index of the stream's kept row,
 * within its window [row_start[s], row_start[s+1]), or -1 to keep the stream
 * as it is; any other value, or a layout that breaks gdn_recur_log's rules,
 * skips the stream.  The kept path (the row and its ancestors, root first) is
 * replayed onto state, and the path's last three raw rows from qkv,
 * continuing into the old tail, become conv_tail.  row_start, parent, qkv and
 * the log are those of the gdn_recur_log call.  The result equals, bit for
 * bit, gdn_commit of the same row after gdn_recur_window / gdn_recur_tree.
 */
int gdn_commit_replay(const gdn_shape *shape, int32_t n_streams, int32_t total_rows,
                      int32_t max_rows, const int32_t *row_start, const int32_t *parent,
                      const int32_t *accept_row, const uint16_t *qkv, const float *log_alpha,
                      const float *log_delta, const float *log_key, uint16_t *conv_tail,
                      float *state, void *stream);

/*
 * Bytes of device workspace gdn_prefill_chunked needs for n_seqs prompts of
 * total_rows rows in all (0 if the shape is refused).
 */
size_t gdn_prefill_workspace_bytes(const gdn_shape *shape, int32_t n_seqs, int32_t total_rows);

/*
 * Prompt passes of several prompts packed in one call (prompts that arrive
 * together share one pass: page "perf(qwen27 cuda): reduce repeated-prompt
 * TTFT", commit note on the lane host admitting every queued request), in
 * the chunkwise WY form with chunks of 64 rows, updating each prompt's state
 * and tail in place.  Chunks never cross prompts.  Geometry: dk == dv == 128
 * and hv / hk <= 8 (GDN_EUNSUPPORTED otherwise).
 *   seq_start [n+1] int32, device: 0 <= seq_start[s] <= seq_start[s+1] <= total_rows
 *   max_len   a bound on every prompt's length (sizes the launch)
 *   qkv [total_rows][C] bf16; a, b [total_rows][hv] bf16
 *   conv_tail [n][3][C] bf16 in/out; state [n][hv][dk][dv] fp32 in/out
 *   out [total_rows][hv][dv] fp32
 *   workspace: device memory of at least gdn_prefill_workspace_bytes()
 * Results match the row-by-row recurrence within the rounding of its bf16
 * matrix-core operands; they are not bitwise equal to one-row steps.
 */
int gdn_prefill_chunked(const gdn_shape *shape, const gdn_params *params, int32_t n_seqs,
                        int32_t total_rows, int32_t max_len, const int32_t *seq_start,
                        const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                        uint16_t *conv_tail, float *state, float *out, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * gdn_prefill_chunked with its workspace in a fixed device array of
 * GDN_PREFILL_SCRATCH_BYTES (128 MiB) that the library holds on every GPU it
 * runs on until the process ends.  Same arguments as gdn_prefill_chunked
 * without the workspace, and bit for bit the same results.  Allocates
 * nothing.
 *  - A pass whose workspace (gdn_prefill_workspace_bytes) exceeds the array
 *    is refused with GDN_EWORKSPACE before anything is launched: at 48 value
 *    heads of 128 that is a pass of more than about 43 chunks of 64 rows
 *    (one prompt of 2,752 rows).
 *    Longer prompts can be passed in pieces cut at multiples of 64 rows,
 *    which give the same bits as one pass.
 *  - `stream` must belong to the calling thread's current device; the
 *    array's address on that device is looked up on the first call there.
 *  - Every call on a GPU shares that GPU's array.  A pass writes every byte
 *    of it that it reads, so nothing has to be cleared between calls, but
 *    calls that overlap on one GPU (on different streams, or from threads
 *    without ordering) race and give undefined results.
 */
#define GDN_PREFILL_SCRATCH_BYTES (128u * 1024u * 1024u)
int gdn_prefill_chunked_noalloc(const gdn_shape *shape, const gdn_params *params, int32_t n_seqs,
                                int32_t total_rows, int32_t max_len, const int32_t *seq_start,
                                const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                                uint16_t *conv_tail, float *state, float *out, void *stream);

/*
 * The in-projection before the mixer: its packed rows qkv and gate inputs a,
 * b from hidden rows x, y = x W^T, with W in affine 4-bit form (the
 * projections of the MLX affine 4-bit checkpoint run through affine-4
 * kernels: page "perf(qwen3_5 cuda): deliver the first token before
 * drafting", note on that checkpoint; the format read as MLX's affine
 * quantisation).  Output features are [qkv (C) | a (hv) | b (hv)], C =
 * 2*hk*dk + hv*dv; weight w[n][k] = scale[n][k/group] * q[n][k] +
 * bias[n][k/group].  Weights are repacked once (at load) into a tiled layout
 * for these kernels: gdn_inproj_pack_affine4.
 *
 * gdn_inproj_padded_features: NP = 16 * ceil((C + 2 hv) / 16), or -1 for a
 * bad shape.
 *
 * gdn_inproj_pack_affine4: MLX layout in, tiled layout out (device arrays,
 * 16-byte aligned, all on `stream`):
 *   wq     [C + 2 hv][hidden/8] packed codes: code j of word w (bits
 *          4j..4j+3) is q[n][8w + j]
 *   scales, biases [C + 2 hv][hidden/group] bf16
 *   wq_tiled [NP * hidden / 8] words; scales_tiled, biases_tiled
 *          [NP * hidden / group] bf16 (the padded features get zeros)
 *
 * gdn_inproj_affine4:
 *   x      [rows][hidden] bf16, device, 16-byte aligned
 *   wq_tiled, scales_tiled, biases_tiled from gdn_inproj_pack_affine4
 *   qkv    [rows][C] bf16 out (16-byte aligned); a, b [rows][hv] bf16 out
 * hidden must be a multiple of 128 and group_size 32, 64 or 128
 * (GDN_EUNSUPPORTED otherwise).  Weights are rounded to bf16 before the
 * matrix-core products, which accumulate in fp32; outputs are rounded to
 * bf16.  rows == 0 does nothing.
 */
int32_t gdn_inproj_padded_features(const gdn_shape *shape);
int gdn_inproj_pack_affine4(const gdn_shape *shape, int32_t hidden, int32_t group_size, const uint32_t *wq,
                            const uint16_t *scales, const uint16_t *biases, uint32_t *wq_tiled,
                            uint16_t *scales_tiled, uint16_t *biases_tiled, void *stream);
int gdn_inproj_affine4(const gdn_shape *shape, int32_t rows, int32_t hidden, int32_t group_size,
                       const uint16_t *x, const uint32_t *wq_tiled, const uint16_t *scales_tiled,
                       const uint16_t *biases_tiled, uint16_t *qkv, uint16_t *a, uint16_t *b, void *stream);

/*
 * Host-side check of a window or tree layout (HOST copies of row_start and,
 * for trees, parent; parent may be NULL for chains).  Returns GDN_OK or
 * GDN_EINVAL with gdn_last_error() naming the first broken rule.
 */
int gdn_check_layout(int32_t n_streams, int32_t total_rows, int32_t max_rows,
                     const int32_t *row_start_host, const int32_t *parent_host);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDN_H */
