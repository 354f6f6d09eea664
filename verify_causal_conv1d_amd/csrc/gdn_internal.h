// Internal declarations shared by libgdn's host layer and its kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

enum RowsMode : int32_t {
    MODE_WINDOW = 0,  // chain windows, every row recorded or logged
    MODE_TREE = 1,    // tree windows, every row recorded or logged
    MODE_STEP = 2,    // one row per stream, state and tail updated in place
};

// Everything one launch of the row kernel needs (passed by value).
struct RowsArgs {
    int32_t hk, hv, dk, dv, C;
    int32_t r;          // value heads per key head
    int32_t vpw;        // value heads handled by one workgroup (divides r)
    int32_t cs;         // workgroups sharing a value head's dv/32 column tiles (1 unless vpw == 1)
    int32_t n_streams, total_rows, max_rows;
    int32_t mode;
    const int32_t *row_start;  // [n+1] (unused in MODE_STEP)
    const int32_t *parent;     // [total_rows] (MODE_TREE only)
    const uint16_t *qkv, *a, *b;
    const float *conv_w, *a_log, *dt_bias;
    const uint16_t *tail_in;
    uint16_t *tail_out;        // MODE_STEP: in place (== tail_in)
    const float *state_in;
    float *state_out;          // MODE_STEP: in place (== state_in)
    float *out;
    uint16_t *tail_snap;       // [total_rows][3][C] (window / tree, recorded)
    float *state_snap;         // [total_rows][hv][dk][dv] (window / tree, recorded)
    int32_t logged;            // window / tree: log each row instead of recording it
    float *log_alpha;          // [total_rows][hv]      decay
    float *log_delta;          // [total_rows][hv][dv]  write
    float *log_key;            // [total_rows][hk][dk]  khat
    int32_t cache_rows;        // MODE_TREE: dk / 32 when a quarter of each lane's state rows stays in LDS for the reloads, else 0
};

struct CommitArgs {
    int32_t n_streams, total_rows;
    size_t state_elems;   // hv * dk * dv
    size_t tail_elems;    // 3 * C
    const int32_t *row_start;   // [n+1]: the accepted row must lie in its stream's window
    const int32_t *accept;
    const uint16_t *tail_snap;
    const float *state_snap;
    uint16_t *tail;
    float *state;
};

// Commit by replay of the logged kept paths.
struct ReplayArgs {
    int32_t hk, hv, dk, dv, C;
    int32_t n_streams, total_rows, max_rows;
    const int32_t *row_start;
    const int32_t *parent;     // NULL: chains
    const int32_t *accept;
    const uint16_t *qkv;
    const float *log_alpha, *log_delta, *log_key;
    uint16_t *tail;
    float *state;
};

// Rows a verify window may hold.
constexpr int kMaxWindowRows = 16;

// LDS one row-kernel workgroup may use (gfx950 has 160 KiB a CU).
constexpr size_t kRowsMaxLds = 160 * 1024;

// Threads of one row-kernel workgroup and its dynamic LDS bytes.
int rows_block_threads(const RowsArgs &A);
size_t rows_lds_bytes(const RowsArgs &A);
// LDS of a row workgroup before the trees' state-row cache, which starts there
__host__ __device__ inline size_t rows_state_cache_offset(const RowsArgs &A)
{
    const size_t nch = 2 * (size_t)A.dk + (size_t)A.vpw * A.dv;
    const size_t mr = A.max_rows;
    const size_t base = sizeof(float) * mr * nch                  // act
           + sizeof(float) * 4 * nch                 // conv weights
           + sizeof(uint16_t) * (3 + mr) * nch       // raw rows
           + (A.logged || A.mode == MODE_TREE ? sizeof(float) * mr * A.vpw * A.dv : 0)   // writes kept for replays
           + sizeof(float) * 2 * mr * A.vpw          // gates
           + sizeof(int) * (7 * mr + 1);             // ancestors, order, subtree sizes, ancestor masks, flag
    return (base + 15) & ~(size_t)15;
}
int rows_cache_rows_that_fit(const RowsArgs &A);   // dk / 32 for trees whose LDS has room, else 0

hipError_t launch_step(const RowsArgs &A, hipStream_t stream);   // MODE_STEP, max_rows = 1, vpw = r
hipError_t launch_rows(const RowsArgs &A, hipStream_t stream);
hipError_t launch_commit(const CommitArgs &A, hipStream_t stream);
hipError_t launch_replay(const ReplayArgs &A, hipStream_t stream);

}  // namespace gdn
