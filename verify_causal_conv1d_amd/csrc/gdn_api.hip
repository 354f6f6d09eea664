// Host side of libgdn's C ABI: argument checks, launch configuration, and
// launches on the caller's stream.  Declarations and contracts are in
// include/libgdn.h.  Nothing here allocates device memory or keeps state
// between calls.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/libgdn.h"
#include "gdn_internal.h"
#include "gdn_inproj.h"
#include "gdn_prefill.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const gdn_shape *s)
{
    if (!s) return fail(GDN_EINVAL, "shape is NULL");
    if (s->hk <= 0 || s->hv <= 0 || s->dk <= 0 || s->dv <= 0 || s->conv_width <= 0)
        return fail(GDN_EINVAL, "shape sizes must be positive (hk=%d hv=%d dk=%d dv=%d conv_width=%d)",
                    s->hk, s->hv, s->dk, s->dv, s->conv_width);
    if (s->hv % s->hk != 0)
        return fail(GDN_EINVAL, "hv (%d) must be a multiple of hk (%d)", s->hv, s->hk);
    if (s->conv_width != 4) return fail(GDN_EUNSUPPORTED, "conv_width %d: only 4 is supported", s->conv_width);
    if (s->dk != 64 && s->dk != 128) return fail(GDN_EUNSUPPORTED, "dk %d: only 64 and 128 are supported", s->dk);
    if (s->dv != 64 && s->dv != 128) return fail(GDN_EUNSUPPORTED, "dv %d: only 64 and 128 are supported", s->dv);
    const long long C = 2LL * s->hk * s->dk + (long long)s->hv * s->dv;
    if (C > (1LL << 24)) return fail(GDN_EUNSUPPORTED, "too many channels (%lld)", C);
    return GDN_OK;
}

int check_params(const gdn_params *p)
{
    if (!p) return fail(GDN_EINVAL, "params is NULL");
    if (!p->conv_w || !p->a_log || !p->dt_bias) return fail(GDN_EINVAL, "a parameter pointer is NULL");
    if (!aligned16(p->conv_w)) return fail(GDN_EINVAL, "conv_w must be 16-byte aligned");
    return GDN_OK;
}

#define REQUIRE_PTR(p)                                                                  \
    do {                                                                                \
        if (!(p)) return fail(GDN_EINVAL, "%s is NULL", #p);                            \
        if (!aligned16(p)) return fail(GDN_EINVAL, "%s must be 16-byte aligned", #p);   \
    } while (0)

// Value heads per workgroup: the largest divisor of r whose workgroup stays
// within 16 waves (1024 threads; a wave holds 32 state columns of a head).
// LIBGDN_HEADS_PER_BLOCK overrides it (a tuning knob; it must divide r and
// fit the limit).
int heads_per_block(int r, int dv)
{
    const int waves_per_head = dv / 32;
    int best = 1;
    for (int v = 1; v <= r; ++v)
        if (r % v == 0 && v * waves_per_head <= 16) best = v;
    if (const char *e = getenv("LIBGDN_HEADS_PER_BLOCK")) {
        const int v = atoi(e);
        if (v >= 1 && r % v == 0 && v * waves_per_head <= 16) best = v;
    }
    return best;
}

// Workgroups of a verify pass.  A launch with few streams would leave most
// CUs idle and put every row's snapshot stores of a key head through one CU:
// then each value head gets its own workgroups, cs of them sharing its dv/32
// column tiles, as many as keep the launch within the chip's 256 CUs.  The
// per-lane arithmetic is the same for every split, so results do not depend
// on it.  Otherwise the widest workgroups heads_per_block allows.
void split_columns(gdn::RowsArgs &A, int n_streams)
{
    const int tiles = A.dv / 32;
    A.vpw = heads_per_block(A.r, A.dv);
    A.cs = 1;
    if (getenv("LIBGDN_HEADS_PER_BLOCK")) return;
    for (int cs = tiles; cs >= 2; cs /= 2) {
        if (tiles % cs == 0 && (long long)n_streams * A.hv * cs <= 256) {
            A.vpw = 1;
            A.cs = cs;
            return;
        }
    }
}

gdn::RowsArgs rows_args(const gdn_shape *s, const gdn_params *p)
{
    gdn::RowsArgs A = {};
    A.hk = s->hk;
    A.hv = s->hv;
    A.dk = s->dk;
    A.dv = s->dv;
    A.C = 2 * s->hk * s->dk + s->hv * s->dv;
    A.r = s->hv / s->hk;
    A.vpw = 1;
    A.cs = 1;
    A.conv_w = p->conv_w;
    A.a_log = p->a_log;
    A.dt_bias = p->dt_bias;
    return A;
}

int launched(hipError_t e)
{
    if (e != hipSuccess) return fail(GDN_EHIP, "launch failed: %s", hipGetErrorString(e));
    g_err[0] = '\0';
    return GDN_OK;
}

// What a verify pass leaves besides o: every row's recorded tail and state,
// or (logged) every row's decay, write and key.
struct PassOutputs {
    uint16_t *tail_snap;
    float *state_snap;
    bool logged;
    float *log_alpha, *log_delta, *log_key;
};

int window_or_tree(const gdn_shape *shape, const gdn_params *params, int32_t n_streams,
                   int32_t total_rows, int32_t max_rows, const int32_t *row_start,
                   const int32_t *parent, bool tree, const uint16_t *qkv, const uint16_t *a,
                   const uint16_t *b, const uint16_t *conv_tail, const float *state, float *out,
                   const PassOutputs &po, void *stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    rc = check_params(params);
    if (rc) return rc;
    if (n_streams < 0) return fail(GDN_EINVAL, "n_streams %d is negative", n_streams);
    if (total_rows < 0) return fail(GDN_EINVAL, "total_rows %d is negative", total_rows);
    if (max_rows < 1 || max_rows > GDN_MAX_WINDOW_ROWS)
        return fail(GDN_EINVAL, "max_rows %d is outside 1..%d", max_rows, GDN_MAX_WINDOW_ROWS);
    if ((long long)total_rows > (long long)n_streams * max_rows)
        return fail(GDN_EINVAL, "total_rows %d exceeds n_streams * max_rows", total_rows);
    if (n_streams == 0 || total_rows == 0) {
        g_err[0] = '\0';
        return GDN_OK;  // nothing to do
    }
    if (!row_start) return fail(GDN_EINVAL, "row_start is NULL");
    if (tree && !parent) return fail(GDN_EINVAL, "parent is NULL");
    REQUIRE_PTR(qkv);
    if (!a || !b) return fail(GDN_EINVAL, "a or b is NULL");
    REQUIRE_PTR(conv_tail);
    REQUIRE_PTR(state);
    REQUIRE_PTR(out);
    if (po.logged) {
        const float *log_alpha = po.log_alpha, *log_delta = po.log_delta, *log_key = po.log_key;
        REQUIRE_PTR(log_alpha);
        REQUIRE_PTR(log_delta);
        REQUIRE_PTR(log_key);
    } else {
        const uint16_t *tail_snap = po.tail_snap;
        const float *state_snap = po.state_snap;
        REQUIRE_PTR(tail_snap);
        REQUIRE_PTR(state_snap);
    }
    gdn::RowsArgs A = rows_args(shape, params);
    split_columns(A, n_streams);
    A.n_streams = n_streams;
    A.total_rows = total_rows;
    A.max_rows = max_rows;
    A.mode = tree ? gdn::MODE_TREE : gdn::MODE_WINDOW;
    A.row_start = row_start;
    A.parent = parent;
    A.qkv = qkv;
    A.a = a;
    A.b = b;
    A.tail_in = conv_tail;
    A.state_in = state;
    A.out = out;
    A.tail_snap = po.tail_snap;
    A.state_snap = po.state_snap;
    A.logged = po.logged ? 1 : 0;
    A.log_alpha = po.log_alpha;
    A.log_delta = po.log_delta;
    A.log_key = po.log_key;
    if ((long long)n_streams * A.hk * (A.r / A.vpw) * A.cs > 0x7fffffffLL)
        return fail(GDN_EUNSUPPORTED, "too many streams for one launch");
    if (gdn::rows_lds_bytes(A) > gdn::kRowsMaxLds)
        return fail(GDN_EUNSUPPORTED, "window needs %zu bytes of LDS", gdn::rows_lds_bytes(A));
    // trees keep a quarter of the stream's state in LDS where it fits beside
    // the rest, so that their reloads read less from memory
    A.cache_rows = gdn::rows_cache_rows_that_fit(A);
    return launched(gdn::launch_rows(A, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char *gdn_status_name(int status)
{
    switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_EINVAL: return "GDN_EINVAL";
    case GDN_EUNSUPPORTED: return "GDN_EUNSUPPORTED";
    case GDN_EWORKSPACE: return "GDN_EWORKSPACE";
    case GDN_EHIP: return "GDN_EHIP";
    default: return "GDN_UNKNOWN";
    }
}

const char *gdn_last_error(void) { return g_err; }

int32_t gdn_channels(const gdn_shape *shape)
{
    if (check_shape(shape) != GDN_OK) return -1;
    return 2 * shape->hk * shape->dk + shape->hv * shape->dv;
}

int gdn_conv_step(const gdn_shape *shape, const gdn_params *params, int32_t n_streams,
                  const uint16_t *qkv, const uint16_t *a, const uint16_t *b, uint16_t *conv_tail,
                  float *state, float *out, void *stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    rc = check_params(params);
    if (rc) return rc;
    if (n_streams < 0) return fail(GDN_EINVAL, "n_streams %d is negative", n_streams);
    const int r = shape->hv / shape->hk;
    if (r * (shape->dv / 32) > 16)
        return fail(GDN_EUNSUPPORTED, "one-row steps need (hv/hk) * dv <= 512 (got %d * %d)", r, shape->dv);
    if (n_streams == 0) {
        g_err[0] = '\0';
        return GDN_OK;
    }
    REQUIRE_PTR(qkv);
    if (!a || !b) return fail(GDN_EINVAL, "a or b is NULL");
    REQUIRE_PTR(conv_tail);
    REQUIRE_PTR(state);
    REQUIRE_PTR(out);
    gdn::RowsArgs A = rows_args(shape, params);
    A.vpw = A.r;  // one workgroup per key head: it alone reads and rewrites those tail channels
    A.cs = 1;
    A.n_streams = n_streams;
    A.total_rows = n_streams;
    A.max_rows = 1;
    A.mode = gdn::MODE_STEP;
    A.qkv = qkv;
    A.a = a;
    A.b = b;
    A.tail_in = conv_tail;
    A.tail_out = conv_tail;
    A.state_in = state;
    A.state_out = state;
    A.out = out;
    return launched(gdn::launch_step(A, static_cast<hipStream_t>(stream)));
}

int gdn_recur_window(const gdn_shape *shape, const gdn_params *params, int32_t n_streams,
                     int32_t total_rows, int32_t max_rows, const int32_t *row_start,
                     const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                     const uint16_t *conv_tail, const float *state, float *out,
                     uint16_t *tail_snap, float *state_snap, void *stream)
{
    const PassOutputs po = {tail_snap, state_snap, false, nullptr, nullptr, nullptr};
    return window_or_tree(shape, params, n_streams, total_rows, max_rows, row_start, nullptr, false,
                          qkv, a, b, conv_tail, state, out, po, stream);
}

int gdn_recur_tree(const gdn_shape *shape, const gdn_params *params, int32_t n_streams,
                   int32_t total_rows, int32_t max_rows, const int32_t *row_start,
                   const int32_t *parent, const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                   const uint16_t *conv_tail, const float *state, float *out, uint16_t *tail_snap,
                   float *state_snap, void *stream)
{
    const PassOutputs po = {tail_snap, state_snap, false, nullptr, nullptr, nullptr};
    return window_or_tree(shape, params, n_streams, total_rows, max_rows, row_start, parent, true,
                          qkv, a, b, conv_tail, state, out, po, stream);
}

int gdn_recur_log(const gdn_shape *shape, const gdn_params *params, int32_t n_streams,
                  int32_t total_rows, int32_t max_rows, const int32_t *row_start, const int32_t *parent,
                  const uint16_t *qkv, const uint16_t *a, const uint16_t *b, const uint16_t *conv_tail,
                  const float *state, float *out, float *log_alpha, float *log_delta, float *log_key,
                  void *stream)
{
    const PassOutputs po = {nullptr, nullptr, true, log_alpha, log_delta, log_key};
    return window_or_tree(shape, params, n_streams, total_rows, max_rows, row_start, parent,
                          parent != nullptr, qkv, a, b, conv_tail, state, out, po, stream);
}

int gdn_commit_replay(const gdn_shape *shape, int32_t n_streams, int32_t total_rows, int32_t max_rows,
                      const int32_t *row_start, const int32_t *parent, const int32_t *accept_row,
                      const uint16_t *qkv, const float *log_alpha, const float *log_delta,
                      const float *log_key, uint16_t *conv_tail, float *state, void *stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (n_streams < 0) return fail(GDN_EINVAL, "n_streams %d is negative", n_streams);
    if (total_rows < 0) return fail(GDN_EINVAL, "total_rows %d is negative", total_rows);
    if (max_rows < 1 || max_rows > GDN_MAX_WINDOW_ROWS)
        return fail(GDN_EINVAL, "max_rows %d is outside 1..%d", max_rows, GDN_MAX_WINDOW_ROWS);
    if ((long long)n_streams * shape->hv > 0x7fffffffLL)
        return fail(GDN_EUNSUPPORTED, "too many streams for one launch");
    if (n_streams == 0 || total_rows == 0) {
        g_err[0] = '\0';
        return GDN_OK;
    }
    if (!row_start) return fail(GDN_EINVAL, "row_start is NULL");
    if (!accept_row) return fail(GDN_EINVAL, "accept_row is NULL");
    REQUIRE_PTR(qkv);
    REQUIRE_PTR(log_alpha);
    REQUIRE_PTR(log_delta);
    REQUIRE_PTR(log_key);
    REQUIRE_PTR(conv_tail);
    REQUIRE_PTR(state);
    gdn::ReplayArgs A = {};
    A.hk = shape->hk;
    A.hv = shape->hv;
    A.dk = shape->dk;
    A.dv = shape->dv;
    A.C = 2 * shape->hk * shape->dk + shape->hv * shape->dv;
    A.n_streams = n_streams;
    A.total_rows = total_rows;
    A.max_rows = max_rows;
    A.row_start = row_start;
    A.parent = parent;
    A.accept = accept_row;
    A.qkv = qkv;
    A.log_alpha = log_alpha;
    A.log_delta = log_delta;
    A.log_key = log_key;
    A.tail = conv_tail;
    A.state = state;
    return launched(gdn::launch_replay(A, static_cast<hipStream_t>(stream)));
}

int gdn_commit(const gdn_shape *shape, int32_t n_streams, int32_t total_rows,
               const int32_t *row_start, const int32_t *accept_row, const uint16_t *tail_snap,
               const float *state_snap, uint16_t *conv_tail, float *state, void *stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (n_streams < 0) return fail(GDN_EINVAL, "n_streams %d is negative", n_streams);
    if (total_rows < 0) return fail(GDN_EINVAL, "total_rows %d is negative", total_rows);
    if (n_streams > 65535) return fail(GDN_EUNSUPPORTED, "at most 65535 streams a commit");
    if (n_streams == 0 || total_rows == 0) {
        g_err[0] = '\0';
        return GDN_OK;
    }
    if (!row_start) return fail(GDN_EINVAL, "row_start is NULL");
    if (!accept_row) return fail(GDN_EINVAL, "accept_row is NULL");
    REQUIRE_PTR(tail_snap);
    REQUIRE_PTR(state_snap);
    REQUIRE_PTR(conv_tail);
    REQUIRE_PTR(state);
    gdn::CommitArgs A = {};
    A.n_streams = n_streams;
    A.total_rows = total_rows;
    A.state_elems = (size_t)shape->hv * shape->dk * shape->dv;
    A.tail_elems = 3 * (size_t)(2 * shape->hk * shape->dk + shape->hv * shape->dv);
    A.row_start = row_start;
    A.accept = accept_row;
    A.tail_snap = tail_snap;
    A.state_snap = state_snap;
    A.tail = conv_tail;
    A.state = state;
    return launched(gdn::launch_commit(A, static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_workspace_bytes(const gdn_shape *shape, int32_t n_seqs, int32_t total_rows)
{
    if (check_shape(shape) != GDN_OK || n_seqs < 0 || total_rows < 0) return 0;
    return gdn::prefill_workspace_bytes(shape->hk, shape->hv, shape->dk, shape->dv, n_seqs, total_rows);
}

}  // extern "C"

namespace {

// Checks of a prompt pass's host-visible arguments; fills P (all but the
// workspace) and the workspace bytes the pass needs.  GDN_OK with
// P.total_rows == 0 means there is nothing to do.
int prefill_checked(const gdn_shape *shape, const gdn_params *params, int32_t n_seqs, int32_t total_rows,
                    int32_t max_len, const int32_t *seq_start, const uint16_t *qkv, const uint16_t *a,
                    const uint16_t *b, uint16_t *conv_tail, float *state, float *out, gdn::PrefillArgs &P,
                    size_t &need)
{
    P = gdn::PrefillArgs{};
    need = 0;
    int rc = check_shape(shape);
    if (rc) return rc;
    rc = check_params(params);
    if (rc) return rc;
    if (n_seqs < 0) return fail(GDN_EINVAL, "n_seqs %d is negative", n_seqs);
    if (total_rows < 0) return fail(GDN_EINVAL, "total_rows %d is negative", total_rows);
    if (max_len < 0) return fail(GDN_EINVAL, "max_len %d is negative", max_len);
    if (n_seqs == 0 || total_rows == 0) {
        g_err[0] = '\0';
        return GDN_OK;
    }
    if (max_len == 0) return fail(GDN_EINVAL, "max_len is 0 but total_rows is %d", total_rows);
    if ((long long)max_len > total_rows) return fail(GDN_EINVAL, "max_len exceeds total_rows");
    if (!gdn::prefill_supported(shape->hk, shape->hv, shape->dk, shape->dv))
        return fail(GDN_EUNSUPPORTED, "chunked prompt passes need dk == dv == 128 and hv/hk <= 8");
    if (!seq_start) return fail(GDN_EINVAL, "seq_start is NULL");
    REQUIRE_PTR(qkv);
    if (!a || !b) return fail(GDN_EINVAL, "a or b is NULL");
    REQUIRE_PTR(conv_tail);
    REQUIRE_PTR(state);
    REQUIRE_PTR(out);
    need = gdn::prefill_workspace_bytes(shape->hk, shape->hv, shape->dk, shape->dv, n_seqs, total_rows);
    P.hk = shape->hk;
    P.hv = shape->hv;
    P.dk = shape->dk;
    P.dv = shape->dv;
    P.C = 2 * shape->hk * shape->dk + shape->hv * shape->dv;
    P.n_seqs = n_seqs;
    P.total_rows = total_rows;
    P.max_len = max_len;
    P.seq_start = seq_start;
    P.qkv = qkv;
    P.a = a;
    P.b = b;
    P.conv_w = params->conv_w;
    P.a_log = params->a_log;
    P.dt_bias = params->dt_bias;
    P.conv_tail = conv_tail;
    P.state = state;
    P.out = out;
    return GDN_OK;
}

// The fixed workspace of gdn_prefill_chunked_noalloc: one copy on every GPU
// the library runs on, held until the process ends.  In host code this name
// is only a stand-in for the device array; its device address on each GPU
// comes from hipGetSymbolAddress, once per device, and only that address is
// ever passed to a kernel.
__device__ __align__(256) unsigned char scratch[GDN_PREFILL_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device (looked up on the
// device's first call, with that device current).
int scratch_on_current_device(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GDN_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GDN_EHIP, "scratch array address on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_prefill_chunked(const gdn_shape *shape, const gdn_params *params, int32_t n_seqs,
                        int32_t total_rows, int32_t max_len, const int32_t *seq_start,
                        const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                        uint16_t *conv_tail, float *state, float *out, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    gdn::PrefillArgs P;
    size_t need = 0;
    int rc = prefill_checked(shape, params, n_seqs, total_rows, max_len, seq_start, qkv, a, b, conv_tail,
                             state, out, P, need);
    if (rc || P.total_rows == 0) return rc;
    if (!workspace || workspace_bytes < need)
        return fail(GDN_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(GDN_EINVAL, "workspace must be 16-byte aligned");
    P.workspace = workspace;
    return launched(gdn::launch_prefill(P, static_cast<hipStream_t>(stream)));
}

int gdn_prefill_chunked_noalloc(const gdn_shape *shape, const gdn_params *params, int32_t n_seqs,
                                int32_t total_rows, int32_t max_len, const int32_t *seq_start,
                                const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                                uint16_t *conv_tail, float *state, float *out, void *stream)
{
    gdn::PrefillArgs P;
    size_t need = 0;
    int rc = prefill_checked(shape, params, n_seqs, total_rows, max_len, seq_start, qkv, a, b, conv_tail,
                             state, out, P, need);
    if (rc || P.total_rows == 0) return rc;
    if (need > (size_t)GDN_PREFILL_SCRATCH_BYTES)
        return fail(GDN_EWORKSPACE,
                    "prompt pass needs %zu bytes of workspace, over the fixed %zu: pass the prompts in "
                    "pieces cut at multiples of 64 rows, or call gdn_prefill_chunked",
                    need, (size_t)GDN_PREFILL_SCRATCH_BYTES);
    void *ws = nullptr;
    rc = scratch_on_current_device(&ws);
    if (rc) return rc;
    P.workspace = ws;
    return launched(gdn::launch_prefill(P, static_cast<hipStream_t>(stream)));
}

int gdn_inproj_affine4(const gdn_shape *shape, int32_t rows, int32_t hidden, int32_t group_size,
                       const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                       const uint16_t *biases, uint16_t *qkv, uint16_t *a, uint16_t *b, void *stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (rows < 0) return fail(GDN_EINVAL, "rows %d is negative", rows);
    if (hidden <= 0 || hidden % 128 != 0)
        return fail(GDN_EUNSUPPORTED, "hidden %d: a positive multiple of 128 is needed", hidden);
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(GDN_EUNSUPPORTED, "group_size %d: 32, 64 or 128 is supported", group_size);
    const long long features = gdn_inproj_padded_features(shape);
    if ((long long)rows * hidden > 0x7fffffffLL || features * (hidden / 8) > 0x7fffffffLL)
        return fail(GDN_EUNSUPPORTED, "projection too large for one call");
    if (rows == 0) {
        g_err[0] = '\0';
        return GDN_OK;
    }
    REQUIRE_PTR(x);
    REQUIRE_PTR(wq);
    if (!scales || !biases) return fail(GDN_EINVAL, "scales or biases is NULL");
    REQUIRE_PTR(qkv);
    if (!a || !b) return fail(GDN_EINVAL, "a or b is NULL");
    gdn::InprojArgs A = {};
    A.rows = rows;
    A.hidden = hidden;
    A.group = group_size;
    A.channels = 2 * shape->hk * shape->dk + shape->hv * shape->dv;
    A.hv = shape->hv;
    A.x = x;
    A.wq = wq;
    A.scales = scales;
    A.biases = biases;
    A.qkv = qkv;
    A.a = a;
    A.b = b;
    return launched(gdn::launch_inproj(A, static_cast<hipStream_t>(stream)));
}

int32_t gdn_inproj_padded_features(const gdn_shape *shape)
{
    if (check_shape(shape)) return -1;
    const int features = 2 * shape->hk * shape->dk + shape->hv * shape->dv + 2 * shape->hv;
    return 16 * ((features + 15) / 16);
}

int gdn_inproj_pack_affine4(const gdn_shape *shape, int32_t hidden, int32_t group_size, const uint32_t *wq,
                            const uint16_t *scales, const uint16_t *biases, uint32_t *wq_tiled,
                            uint16_t *scales_tiled, uint16_t *biases_tiled, void *stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (hidden <= 0 || hidden % 128 != 0)
        return fail(GDN_EUNSUPPORTED, "hidden %d: a positive multiple of 128 is needed", hidden);
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(GDN_EUNSUPPORTED, "group_size %d: 32, 64 or 128 is supported", group_size);
    const long long np = gdn_inproj_padded_features(shape);
    if (np * (hidden / 8) > 0x7fffffffLL) return fail(GDN_EUNSUPPORTED, "projection too large for one call");
    REQUIRE_PTR(wq);
    if (!scales || !biases) return fail(GDN_EINVAL, "scales or biases is NULL");
    REQUIRE_PTR(wq_tiled);
    if (!scales_tiled || !biases_tiled) return fail(GDN_EINVAL, "scales_tiled or biases_tiled is NULL");
    gdn::InprojPackArgs P = {};
    P.hidden = hidden;
    P.group = group_size;
    P.channels = 2 * shape->hk * shape->dk + shape->hv * shape->dv;
    P.hv = shape->hv;
    P.blocks = (int)(np / 16);
    P.wq = wq;
    P.scales = scales;
    P.biases = biases;
    P.wq_tiled = wq_tiled;
    P.scales_tiled = scales_tiled;
    P.biases_tiled = biases_tiled;
    return launched(gdn::launch_inproj_pack(P, static_cast<hipStream_t>(stream)));
}

int gdn_check_layout(int32_t n_streams, int32_t total_rows, int32_t max_rows,
                     const int32_t *row_start_host, const int32_t *parent_host)
{
    if (n_streams < 0 || total_rows < 0) return fail(GDN_EINVAL, "negative count");
    if (max_rows < 1 || max_rows > GDN_MAX_WINDOW_ROWS)
        return fail(GDN_EINVAL, "max_rows %d is outside 1..%d", max_rows, GDN_MAX_WINDOW_ROWS);
    if (n_streams == 0) return GDN_OK;
    if (!row_start_host) return fail(GDN_EINVAL, "row_start is NULL");
    if (row_start_host[0] < 0) return fail(GDN_EINVAL, "row_start[0] = %d is negative", row_start_host[0]);
    for (int s = 0; s < n_streams; ++s) {
        const int r0 = row_start_host[s], r1 = row_start_host[s + 1];
        if (r1 < r0) return fail(GDN_EINVAL, "row_start decreases at stream %d", s);
        if (r1 > total_rows) return fail(GDN_EINVAL, "stream %d ends past total_rows", s);
        if (r1 - r0 > max_rows) return fail(GDN_EINVAL, "stream %d has %d rows > max_rows %d", s, r1 - r0, max_rows);
        if (parent_host)
            for (int t = 0; t < r1 - r0; ++t) {
                const int p = parent_host[r0 + t];
                if (p < -1 || p >= t)
                    return fail(GDN_EINVAL, "stream %d row %d: parent %d is not in [-1, %d)", s, t, p, t);
            }
    }
    g_err[0] = '\0';
    return GDN_OK;
}

}  // extern "C"
