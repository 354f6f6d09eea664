// Row kernels of libgdn: one-row steps, verify windows and verify trees of the
// gated-delta-rule mixer, plus the commit copy.  gfx950 (CDNA4), wave64.
//
// One workgroup serves one stream and `vpw` value heads of one key head; in a
// launch too small to fill the chip, a share of one value head's column tiles.
//
//   prologue  the raw bf16 rows of the window and the stream's tail (only the
//             workgroup's channels) and the conv weights are staged in LDS
//             with 16-byte loads issued together, and the state tile's loads
//             right behind them, so the prologue pays one global latency and
//             the state streams in while it runs; then causal conv (taps
//             along the row's own branch) + SiLU, 8 channels of a row a
//             thread, from LDS; gates per (row, value head); per row an L2
//             norm of q and of k (q also times dk^-1/2).  Tail snapshots are
//             16-byte copies out of the staged rows.
//   rows      each wave owns 32 columns of one value head's state M = S^T
//             ([dk][dv], dv contiguous).  Lane (c, g) = (lane & 7, lane >> 3)
//             keeps rows [g*dk/8, (g+1)*dk/8) x columns [4c, 4c+4) of the
//             tile in VGPRs for the whole window, so the state crosses HBM
//             once on the way in; the per-row snapshot is written with
//             dwordx4 stores that form full 128-byte row segments.
//             The two dk-sums (M^T k and M^T q) are per-lane partials over the
//             lane's rows, then a butterfly over the eight 8-lane groups: a
//             DPP row rotate, then the gfx950 lane-swap instructions.  No
//             barrier inside the row loop, and no global load except a tree
//             row's reload of the stream's state.  Narrow tiles spread the row loop's
//             fp32 work (four operations per state element and row) over
//             twice the waves of 64-column ones.
//
// Logged windows and trees (page "perf(qwen3_5 cuda): deliver the first token
// before drafting", commit note on tree-shaped verify windows: a verify logs
// its rows' decay, write and key instead of every row's state) record, per
// row, alpha (per value head), khat (per key head) and the write delta with
// M_t = alpha M_p + khat delta^T (per value head), and no snapshot.  A tree
// row (logged or recorded) whose parent is not the row just done rebuilds the
// parent's state: the stream's state reloaded, then the parent's path
// replayed from the decays, writes and keys kept in LDS with the very
// operations that first produced it.  The commit by replay replays the kept
// path the same way, so it reaches, bit for bit, the state a recorded window
// holds for that row.
//
// Every row of every mode runs this same code in the same order, so a window's
// rows equal one-row steps bit for bit and a tree's paths equal chains (the
// pages require window rows to equal one-row steps bit for bit: page
// "perf(qwen3_5 cuda): deliver the first token before drafting", commit note
// on the MLX affine 4-bit checkpoint).  The build disables fp contraction;
// every fused multiply-add below is written out.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferDword3 = 0x00020000;   // buffer resource word 3 (gfx950 raw buffer)

// bf16 number e (0..7) of eight packed in a 16-byte chunk, as fp32
__device__ __forceinline__ float bf16_word(const uint4 &x, int e)
{
    const uint32_t w = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Global channel of local prologue channel `ch`: [q of kh | k of kh | v of
// the workgroup's value heads].
__device__ __forceinline__ int global_channel(const RowsArgs &A, int dk, int kh, int h0, int ch)
{
    if (ch < dk) return kh * dk + ch;
    if (ch < 2 * dk) return A.hk * dk + kh * dk + (ch - dk);
    return 2 * A.hk * dk + h0 * A.dv + (ch - 2 * dk);
}

// One row of the recurrence on a lane's tile m: state rows [grp R, grp R + R)
// of the head (stored form M = S^T), columns col .. col + 3.  krow and qrow
// hold the lane's R entries of k^ and q^.  u = M^T k^ (the lane's rows, then
// across the eight row groups), d = beta (v - alpha u), M <- alpha M + k^ d^T
// with each updated state row stored to dst at once when STORE (so the stores
// issue among the arithmetic; NT: non-temporal), o = M^T q^.  Window rows and
// one-row steps both run this, so they agree bit for bit.
template <int R, bool STORE, bool NT>
__device__ __forceinline__ void row_step(float4 (&m)[R], const float *krow, const float *qrow, const float4 vv,
                                         const float al, const float be, float *dst, const int dv,
                                         float4 &d, float4 &o)
{
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < R; i += 4) {
        const float4 kv = *reinterpret_cast<const float4 *>(krow + i);
        const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u.x = fmaf(m[i + e].x, kk[e], u.x);
            u.y = fmaf(m[i + e].y, kk[e], u.y);
            u.z = fmaf(m[i + e].z, kk[e], u.z);
            u.w = fmaf(m[i + e].w, kk[e], u.w);
        }
    }
    u.x = sum_rows8(u.x);
    u.y = sum_rows8(u.y);
    u.z = sum_rows8(u.z);
    u.w = sum_rows8(u.w);
    d.x = be * (vv.x - al * u.x);
    d.y = be * (vv.y - al * u.y);
    d.z = be * (vv.z - al * u.z);
    d.w = be * (vv.w - al * u.w);
    o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < R; i += 4) {
        const float4 kv = *reinterpret_cast<const float4 *>(krow + i);
        const float4 qv = *reinterpret_cast<const float4 *>(qrow + i);
        const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
        const float qq[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float4 &me = m[i + e];
            me.x = fmaf(kk[e], d.x, al * me.x);
            me.y = fmaf(kk[e], d.y, al * me.y);
            me.z = fmaf(kk[e], d.z, al * me.z);
            me.w = fmaf(kk[e], d.w, al * me.w);
            o.x = fmaf(me.x, qq[e], o.x);
            o.y = fmaf(me.y, qq[e], o.y);
            o.z = fmaf(me.z, qq[e], o.z);
            o.w = fmaf(me.w, qq[e], o.w);
            if (STORE) {
                const f4v val = {me.x, me.y, me.z, me.w};
                if (NT)
                    __builtin_nontemporal_store(val, reinterpret_cast<f4v *>(dst + (size_t)(i + e) * dv));
                else
                    *reinterpret_cast<f4v *>(dst + (size_t)(i + e) * dv) = val;
            }
        }
    }
    o.x = sum_rows8(o.x);
    o.y = sum_rows8(o.y);
    o.z = sum_rows8(o.z);
    o.w = sum_rows8(o.w);
}

template <int DK, bool LOG, bool NT>
__global__ void __launch_bounds__(1024) rows_kernel(const RowsArgs A)
{
    // LOG: a logged window or tree, a template argument so that the recording
    // stores in the row loop carry no branch.  NT: recorded trees, whose
    // snapshots leave with non-temporal stores (chains keep ordinary ones)
    constexpr int R = DK / 8;  // state rows held by one lane
    extern __shared__ float smem[];

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int groups = A.r / A.vpw;
    int bid = blockIdx.x;
    const int part = bid % A.cs;   // which share of the head's column tiles
    bid /= A.cs;
    const int g = bid % groups;
    bid /= groups;
    const int kh = bid % A.hk;
    const int s = bid / A.hk;
    const int h0 = kh * A.r + g * A.vpw;   // first value head of this workgroup

    // ---- layout of this stream's rows (device-side rules; a stream that
    // breaks them is skipped)
    const int r0 = A.row_start[s], r1 = A.row_start[s + 1];
    if (r0 < 0 || r1 < r0 || r1 > A.total_rows || r1 - r0 > A.max_rows) return;
    const int len = r1 - r0;
    if (len == 0) return;

    const int nch = 2 * DK + A.vpw * A.dv;   // channels of this workgroup
    const int mr = A.max_rows;
    // LDS (every 16-byte-accessed array starts 16-byte aligned: nch % 64 == 0)
    float *act = smem;                                              // [mr][nch] conv+SiLU, then q^, k^
    float4 *wl = reinterpret_cast<float4 *>(act + mr * nch);        // [nch] conv weights
    uint16_t *raw = reinterpret_cast<uint16_t *>(wl + nch);         // [3 + mr][nch] raw bf16 rows
    float *dlog = reinterpret_cast<float *>(raw + (3 + mr) * nch);  // [mr][vpw][dv] writes (logged, trees)
    const bool keep_writes = LOG || A.mode == MODE_TREE;
    float *galpha = dlog + (keep_writes ? mr * A.vpw * A.dv : 0);   // [mr][vpw]
    float *gbeta = galpha + mr * A.vpw;                             // [mr][vpw]
    int *anc = reinterpret_cast<int *>(gbeta + mr * A.vpw);         // [mr][4]
    int *order = anc + mr * 4;                                      // [mr] processing order
    int *sub = order + mr;                                          // [mr] subtree sizes, then next free slot
    int *pmask = sub + mr;                                          // [mr] strict ancestors, a bit each
    int *bad = pmask + mr;
    // trees: rows [0, R / 4) of each row wave's tile of the stream's state,
    // [wave][row][lane], for the reloads
    float4 *stc = reinterpret_cast<float4 *>(reinterpret_cast<unsigned char *>(smem) + rows_state_cache_offset(A));

    // ---- this wave's tile of the state
    // The workgroup holds tiles [part * tpw, (part + 1) * tpw) of each of its
    // value heads (cs workgroups share a head's dv / 32 tiles when a launch
    // is too small to fill the chip otherwise; every lane's arithmetic is the
    // same either way).  Waves past the row loop's (vpw value heads of tpw
    // waves each) only help with the prologue and record the tails; their
    // tile index is clamped to a real one and they load no state.
    const int tpw = A.dv / 32 / A.cs;
    const bool row_wave = wave < A.vpw * tpw;
    const int jl = min(wave / tpw, A.vpw - 1);   // local value head
    const int tile = part * tpw + (row_wave ? wave - jl * tpw : 0);
    const int h = h0 + jl;
    const int c4 = lane & 7, grp = lane >> 3;
    const int col = tile * 32 + c4 * 4;
    const size_t head_elems = (size_t)DK * A.dv;
    const size_t lane_off = (size_t)(grp * R) * A.dv + col;
    const float *st_in_head = A.state_in + ((size_t)s * A.hv + h) * head_elems + lane_off;

    // ---- parents and the three nearest ancestors of every row.  anc[t][0]
    // is the parent (whose state row t starts from); anc[t][d] is the source
    // of x_{t-d}: a local row >= 0, or -1, -2, -3 for tail rows 2, 1, 0.
    // A chain has them in closed form (t - 1, then t - d), with its row order
    // and ancestor masks, written without a barrier; a tree's parents are
    // checked and walked.
    const bool tree = A.mode == MODE_TREE;
    if (tree) {
        if (tid == 0) *bad = 0;
        if (tid < len) anc[tid * 4] = A.parent[r0 + tid];
        lds_barrier();
        if (tid < len && (anc[tid * 4] < -1 || anc[tid * 4] >= tid)) *bad = 1;
        lds_barrier();
        if (*bad) return;
        if (tid < len) {
            int i = tid;
#pragma unroll
            for (int d = 1; d <= 3; ++d) {
                i = (i >= 0) ? anc[i * 4] : i - 1;
                anc[tid * 4 + d] = i;
            }
        }
    } else if (tid < len) {
        anc[tid * 4] = tid - 1;
#pragma unroll
        for (int d = 1; d <= 3; ++d) anc[tid * 4 + d] = tid - d;
        order[tid] = tid;
        pmask[tid] = (1 << tid) - 1;
    }
    // Processing order.  A chain runs in row order.  A tree runs in depth-
    // first preorder (children by increasing index): every row still follows
    // its parent, and a row's parent is the row just done except after a
    // leaf, so the parent state is re-read from its snapshot (leaves - 1)
    // times instead of once for every row whose parent is not the row
    // before it.  Each row's arithmetic is the same in any order.
    if (tree && tid == 0) {
        {
            // subtree sizes (parents have smaller indices than children) ...
            for (int i = 0; i < len; ++i) sub[i] = 1;
            for (int i = len - 1; i > 0; --i)
                if (anc[i * 4] >= 0) sub[anc[i * 4]] += sub[i];
            // ... then preorder slots: a row takes its parent's next free slot
            // and reserves its own subtree after it
            int next_root = 0;
            for (int i = 0; i < len; ++i) {
                const int p = anc[i * 4];
                int pos;
                if (p < 0) {
                    pos = next_root;
                    next_root += sub[i];
                } else {
                    pos = sub[p];
                    sub[p] += sub[i];
                }
                order[pos] = i;
                sub[i] = pos + 1;   // from now on: this row's next free slot
            }
        }
        for (int i = 0; i < len; ++i) {
            const int p = anc[i * 4];
            pmask[i] = p >= 0 ? (pmask[p] | (1 << p)) : 0;
        }
    }

    // ---- stage raw rows (tail rows 0..2, then window rows), conv weights and
    // gates.  Raw row 3 + a holds x of local row a (a = -3..-1: the tail).
    // These loads are issued before the state loads: loads retire in order,
    // so the prologue waits only for what it needs.
    const int C = A.C;
    const uint16_t *tail = A.tail_in + (size_t)s * 3 * C;
    const uint16_t *rows = A.qkv + (size_t)r0 * C;
    const int cpr = nch / 8;                     // 16-byte chunks a row
    // ---- tail snapshots: the tail after row t is (x_{t-2}, x_{t-1}, x_t);
    // q/k channels are shared by the key head's workgroups, group 0 records
    // them; of the workgroups that share a head's columns, the first records.
    // With helper waves these leave after the norms, from the helpers alone.
    const bool record_tails = !LOG && part == 0;
    const int row_threads = 64 * A.vpw * tpw;
    const bool late_tails = nthr > row_threads;
    auto tail_snaps = [&](int first, int stride) {
        const int c_first = (g == 0) ? 0 : (2 * DK) / 8;
        const int cw = cpr - c_first;
        for (int idx = first; idx < len * 3 * cw; idx += stride) {
            const int tj = idx / cw;
            const int lc = (c_first + idx - tj * cw) * 8;
            const int t = tj / 3, j = tj - t * 3;
            const int src_row = 3 + (j == 2 ? t : anc[t * 4 + 2 - j]);
            const int gc = global_channel(A, DK, kh, h0, lc);
            *reinterpret_cast<uint4 *>(A.tail_snap + ((size_t)(r0 + t) * 3 + j) * C + gc) =
                *reinterpret_cast<const uint4 *>(raw + src_row * nch + lc);
        }
    };
    float4 m[R];
    {
        // Every load of a batch is issued before any of them is consumed; loads
        // come from clamped indices, unconditionally (the values past the end
        // are not stored), so no branch surrounds them.  Two row chunks and
        // one weight a thread make one batch of a 16-row window at 768
        // threads; longer windows take more.
        const int nchunks = (len + 3) * cpr;
        const int ngates = len * A.vpw;
        auto load_chunk = [&](int idx) -> uint4 {
            idx = min(idx, nchunks - 1);
            const int rr = idx / cpr;
            const int gc = global_channel(A, DK, kh, h0, (idx - rr * cpr) * 8);
            return *reinterpret_cast<const uint4 *>(rr < 3 ? tail + (size_t)rr * C + gc : rows + (size_t)(rr - 3) * C + gc);
        };
        auto put_chunk = [&](int idx, const uint4 &v) {
            if (idx < nchunks) {
                const int rr = idx / cpr;
                *reinterpret_cast<uint4 *>(raw + rr * nch + (idx - rr * cpr) * 8) = v;
            }
        };
        auto load_weight = [&](int ch) -> float4 {
            return *reinterpret_cast<const float4 *>(A.conv_w + (size_t)global_channel(A, DK, kh, h0, min(ch, nch - 1)) * 4);
        };
        auto put_weight = [&](int ch, const float4 &w) {
            if (ch < nch) wl[ch] = w;
        };
        // (a, b, A_log, dt_bias) of gate index gi = (row, local value head)
        auto load_gate = [&](int gi) -> float4 {
            gi = min(gi, ngates - 1);
            const int t = gi / A.vpw;
            const int hh = h0 + (gi - t * A.vpw);
            return make_float4(bf16f(A.a[(size_t)(r0 + t) * A.hv + hh]), bf16f(A.b[(size_t)(r0 + t) * A.hv + hh]),
                               A.a_log[hh], A.dt_bias[hh]);
        };
        auto put_gate = [&](int gi, const float4 &x) {
            if (gi < ngates) {
                // gates: alpha = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b)
                galpha[gi] = decay_f(log_decay(x.x, x.z, x.w));
                gbeta[gi] = sigmoid_f(x.y);
            }
        };
        {
            const uint4 v0 = load_chunk(tid), v1 = load_chunk(nthr + tid);
            const float4 w0 = load_weight(tid);
            const float4 g0 = load_gate(tid);
            // ---- the state tile, requested right behind the first batch and
            // before any of it is consumed, so that the 16 B a lane and row of
            // state stream in while the batch is written to LDS and the conv and
            // norms run.  Helper waves read through a buffer resource of no size
            // (no memory access, zeros): the code has no branch here, so the
            // compiler's memory-counter waits for the batch leave these loads in
            // flight (the counter retires loads in issue order).
            {
                const int wu = __builtin_amdgcn_readfirstlane(wave);
                const int hu = h0 + min(wu / tpw, A.vpw - 1);
                const float *head = A.state_in + ((size_t)s * A.hv + hu) * head_elems;
                const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float *>(head), 0, wu < A.vpw * tpw ? (int)(head_elems * sizeof(float)) : 0, kBufferDword3);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(srs, (int)((lane_off + (size_t)i * A.dv) * sizeof(float)), 0, 0);
                    m[i] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            put_chunk(tid, v0);
            put_chunk(nthr + tid, v1);
            put_weight(tid, w0);
            put_gate(tid, g0);
        }
        for (int base = 2 * nthr, wbase = nthr, gbase = nthr; base < nchunks || wbase < nch || gbase < ngates;
             base += 2 * nthr, wbase += nthr, gbase += nthr) {
            const uint4 v0 = load_chunk(base + tid), v1 = load_chunk(base + nthr + tid);
            const float4 w0 = load_weight(wbase + tid);
            const float4 g0 = load_gate(gbase + tid);
            put_chunk(base + tid, v0);
            put_chunk(base + nthr + tid, v1);
            put_weight(wbase + tid, w0);
            put_gate(gbase + tid, g0);
        }
        lds_barrier();

        // ---- conv + SiLU of every (row, channel), from the staged rows: a
        // thread takes one 16-byte chunk (8 channels) of a row and reads the
        // four raw rows of its taps at once (x_{t-3} .. x_t along the row's
        // branch: raw rows 3 + anc[t][3], 3 + anc[t][2], 3 + anc[t][1], 3 + t;
        // for a chain, rows t .. t + 3)
        for (int idx = tid; idx < cpr * len; idx += nthr) {
            const int t = idx / cpr;
            const int lc = (idx - t * cpr) * 8;
            const int src[4] = {3 + anc[t * 4 + 3], 3 + anc[t * 4 + 2], 3 + anc[t * 4 + 1], 3 + t};
            uint4 xr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xr[j] = *reinterpret_cast<const uint4 *>(raw + src[j] * nch + lc);
            float y8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float4 w = wl[lc + e];
                float y = w.x * bf16_word(xr[0], e);
                y = fmaf(w.y, bf16_word(xr[1], e), y);
                y = fmaf(w.z, bf16_word(xr[2], e), y);
                y = fmaf(w.w, bf16_word(xr[3], e), y);
                y8[e] = silu_f(y);
            }
            float4 *dst = reinterpret_cast<float4 *>(act + t * nch + lc);
            dst[0] = make_float4(y8[0], y8[1], y8[2], y8[3]);
            dst[1] = make_float4(y8[4], y8[5], y8[6], y8[7]);
        }
        if (record_tails && !late_tails) tail_snaps(tid, nthr);
        lds_barrier();

        // ---- L2 norms of q and k per row (q also scaled by dk^-1/2)
        {
            const int nwaves = nthr >> 6;
            const float qscale = 1.0f / sqrtf((float)DK);
            for (int pr = wave; pr < 2 * len; pr += nwaves) {
                const int t = pr >> 1, which = pr & 1;
                float *v = act + t * nch + which * DK;
                const float x0 = v[lane];
                float ss = x0 * x0;
                float x1 = 0.0f;
                if (DK == 128) {
                    x1 = v[lane + 64];
                    ss = fmaf(x1, x1, ss);
                }
                ss = sum_wave(ss);
                float sc = inv_norm_f(ss);
                if (which == 0) sc = sc * qscale;
                v[lane] = x0 * sc;
                if (DK == 128) v[lane + 64] = x1 * sc;
            }
        }
        lds_barrier();
    }

    // ---- the log's decays (this workgroup's value heads) and keys (the key
    // head's workgroup group 0)
    if (LOG && part == 0) {
        for (int idx = tid; idx < len * A.vpw; idx += nthr) {
            const int t = idx / A.vpw;
            A.log_alpha[(size_t)(r0 + t) * A.hv + h0 + (idx - t * A.vpw)] = galpha[idx];
        }
        if (g == 0) {
            for (int idx = tid; idx < len * (DK / 4); idx += nthr) {
                const int t = idx / (DK / 4), i4 = idx - t * (DK / 4);
                *reinterpret_cast<float4 *>(A.log_key + ((size_t)(r0 + t) * A.hk + kh) * DK + 4 * i4) =
                    *reinterpret_cast<const float4 *>(act + t * nch + DK + 4 * i4);
            }
        }
    }

    if (!row_wave) {   // no barrier below
        if (record_tails && late_tails) tail_snaps(tid - row_threads, nthr - row_threads);
        return;
    }

    // The state tile has arrived before the loop starts.  The memory counter
    // also counts stores: left to the compiler, the waits for the tile's loads
    // would sit at the loop's merge point and hold every row until the last
    // row's snapshot stores had completed.
    wait_vmem();

    // ---- the recurrence, row after row, on the tile held in registers.  A
    // tree reads each row's index and parent from LDS one row ahead; a chain
    // has them in closed form (row k, parent k - 1).
    const bool tree_order = A.mode == MODE_TREE;
    // trees keep rows [0, R / 4) of the lane's tile in LDS (cache_rows is 0
    // or R / 4), so a reload reads three quarters of the tile from memory
    constexpr int RC = R / 4;
    const bool cached = tree_order && A.cache_rows != 0;
    float4 *my_stc = stc + (size_t)wave * RC * 64 + lane;
    if (cached && row_wave) {
#pragma unroll
        for (int i = 0; i < RC; ++i) my_stc[i * 64] = m[i];
    }
    int prev = -1;
    int t = tree_order ? order[0] : 0;
    int p = tree_order ? anc[t * 4] : -1;
    for (int k = 0; k < len; ++k) {
        const int kn = min(k + 1, len - 1);
        const int t_next = tree_order ? order[kn] : kn;
        const int p_next = tree_order ? anc[t_next * 4] : kn - 1;
        if (p != prev) {
            // a tree row whose parent is not the row just done: rebuild the
            // parent's state.  The stream's state is reloaded (for p == -1 it
            // is the state wanted; a lane's first R / 4 rows from the copy in
            // LDS when there is one), then the parent's path is replayed from
            // the decays, writes and keys kept in LDS with the very
            // operations that first produced it, so the rebuilt state equals
            // the parent's bit for bit (a recorded snapshot reread instead has
            // left the caches by then, and costs a full read from memory)
            const float *src = st_in_head;
            // the address is formed anew here: kept from the first load of the
            // tile, its 16 row addresses would be held (and spilled) through
            // the prologue
            asm volatile("" : "+v"(src));
            if (cached) {
#pragma unroll
                for (int i = 0; i < RC; ++i) m[i] = my_stc[i * 64];
            } else {
#pragma unroll
                for (int i = 0; i < RC; ++i) m[i] = *reinterpret_cast<const float4 *>(src + (size_t)i * A.dv);
            }
#pragma unroll
            for (int i = RC; i < R; ++i) m[i] = *reinterpret_cast<const float4 *>(src + (size_t)i * A.dv);
            // the loads complete inside the reload, so that rows without one
            // do not wait: a replay uses every loaded row at once, otherwise
            // an explicit wait
            if (p < 0) wait_vmem();
            if (p >= 0) {
                const int path = pmask[p] | (1 << p);
                for (int j = 0; j <= p; ++j) {
                    if (!((path >> j) & 1)) continue;
                    const float *kr = act + j * nch + DK + grp * R;
                    const float aj = galpha[j * A.vpw + jl];
                    const float4 dj = *reinterpret_cast<const float4 *>(dlog + (j * A.vpw + jl) * A.dv + col);
#pragma unroll
                    for (int i = 0; i < R; i += 4) {
                        const float4 kv = *reinterpret_cast<const float4 *>(kr + i);
                        const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float4 &me = m[i + e];
                            me.x = fmaf(kk[e], dj.x, aj * me.x);
                            me.y = fmaf(kk[e], dj.y, aj * me.y);
                            me.z = fmaf(kk[e], dj.z, aj * me.z);
                            me.w = fmaf(kk[e], dj.w, aj * me.w);
                        }
                    }
                }
            }
        }
        const float *qrow = act + t * nch + grp * R;
        const float *krow = act + t * nch + DK + grp * R;

        // delta = beta (v - alpha u);  M <- alpha M + k delta^T;  o = M^T q.
        // The recorded state (a snapshot) leaves each state row as soon as it
        // is updated, so the stores issue among the row's arithmetic.  Chains
        // store through the caches (non-temporal stores measured far slower
        // back to back: 194 vs 152 us on the 16 x 16 verify); trees store
        // non-temporally, which keeps the stream's state cached for their
        // reloads (189 vs 203 us on 16 x 16-node trees)
        const float al = galpha[t * A.vpw + jl];
        const float be = gbeta[t * A.vpw + jl];
        const float4 vv = *reinterpret_cast<const float4 *>(act + t * nch + 2 * DK + jl * A.dv + col);
        const int row = r0 + t;
        float *dst = A.state_snap + ((size_t)row * A.hv + h) * head_elems + lane_off;
        float4 d, o;
        row_step<R, !LOG, NT>(m, krow, qrow, vv, al, be, dst, A.dv, d, o);

        if (grp == 0)
            *reinterpret_cast<float4 *>(A.out + ((size_t)row * A.hv + h) * A.dv + col) = o;
        // the write: to the log, and (logs and trees) to LDS for a later
        // replay by this wave (every lane group holds the same delta)
        if (LOG && grp == 0)
            *reinterpret_cast<float4 *>(A.log_delta + ((size_t)row * A.hv + h) * A.dv + col) = d;
        if (keep_writes && grp == 0) *reinterpret_cast<float4 *>(dlog + (t * A.vpw + jl) * A.dv + col) = d;
        prev = t;
        t = t_next;
        p = p_next;
    }
}

// One-row step in place: workgroup (stream, key head) over the key head's r
// value heads, each value head's dv / 32 column tiles on a wave each.  Each
// input value goes from memory straight to the thread that uses it, with no
// staging through LDS: waves 0 and 1 take the key head's q and k channels in
// the lanes the norm reads them (lane, and lane + 64 for dk = 128), so conv,
// SiLU and the norm run the window path's operations in its order without a
// barrier in between; thread i takes v channel i (the workgroup has at least
// as many threads as v channels).  Each thread rewrites its channels' tail in
// place after reading the old one: no other workgroup reads those channels.
template <int DK>
__global__ void __launch_bounds__(1024) step_kernel(const RowsArgs A)
{
    constexpr int R = DK / 8;  // state rows held by one lane
    extern __shared__ float smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int s = blockIdx.x, kh = blockIdx.y;
    const int vpw = A.r;
    const int h0 = kh * vpw;
    const int C = A.C;
    const int nv = vpw * A.dv;
    float *act = smem;                    // [2 dk + nv]: q^, k^, v of the row
    float *galpha = act + 2 * DK + nv;    // [vpw]
    float *gbeta = galpha + vpw;          // [vpw]
    // wave -> (local value head, 32-column tile): dv / 32 = 2 or 4 tiles a head
    const int tsh = A.dv == 128 ? 2 : 1;
    const bool row_wave = wave < (vpw << tsh);
    const int jl = min(wave >> tsh, vpw - 1);
    const int tile = row_wave ? wave - (jl << tsh) : 0;
    const int h = h0 + jl;
    const int c4 = lane & 7, grp = lane >> 3;
    const int col = tile * 32 + c4 * 4;
    const size_t head_elems = (size_t)DK * A.dv;
    const size_t lane_off = (size_t)(grp * R) * A.dv + col;
    const float *st_in_head = A.state_in + ((size_t)s * A.hv + h) * head_elems + lane_off;
    const uint16_t *tail = A.tail_in + (size_t)s * 3 * C;
    const uint16_t *rows = A.qkv + (size_t)s * C;
    const int r0 = s;
    float4 m[R];
    {
        constexpr int NQ = DK / 64;               // q or k channels a lane
        uint16_t *tl = A.tail_out + (size_t)s * 3 * C;
        uint16_t xq[NQ][4], xv[4] = {0, 0, 0, 0};
        float4 wq[NQ], wv = make_float4(0.f, 0.f, 0.f, 0.f);
        int gq[NQ], gvc = 0;
        const bool qk_wave = wave < 2;
        if (qk_wave) {
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                gq[j] = global_channel(A, DK, kh, h0, wave * DK + lane + 64 * j);
#pragma unroll
                for (int k = 0; k < 3; ++k) xq[j][k] = tail[(size_t)k * C + gq[j]];
                xq[j][3] = rows[gq[j]];
                wq[j] = *reinterpret_cast<const float4 *>(A.conv_w + (size_t)gq[j] * 4);
            }
        }
        if (tid < nv) {
            gvc = global_channel(A, DK, kh, h0, 2 * DK + tid);
#pragma unroll
            for (int k = 0; k < 3; ++k) xv[k] = tail[(size_t)k * C + gvc];
            xv[3] = rows[gvc];
            wv = *reinterpret_cast<const float4 *>(A.conv_w + (size_t)gvc * 4);
        }
        float av = 0.f, bv = 0.f, al = 0.f, db = 0.f;
        if (tid < vpw) {
            av = bf16f(A.a[(size_t)r0 * A.hv + h0 + tid]);
            bv = bf16f(A.b[(size_t)r0 * A.hv + h0 + tid]);
            al = A.a_log[h0 + tid];
            db = A.dt_bias[h0 + tid];
        }
        // the state tile (row waves only): in flight through the prologue
        if (row_wave) {
#pragma unroll
            for (int i = 0; i < R; ++i) m[i] = *reinterpret_cast<const float4 *>(st_in_head + (size_t)i * A.dv);
        }
        if (qk_wave) {
            float x[NQ];
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                float y = wq[j].x * bf16f(xq[j][0]);
                y = fmaf(wq[j].y, bf16f(xq[j][1]), y);
                y = fmaf(wq[j].z, bf16f(xq[j][2]), y);
                y = fmaf(wq[j].w, bf16f(xq[j][3]), y);
                x[j] = silu_f(y);
            }
            float ss = x[0] * x[0];
            if (NQ == 2) ss = fmaf(x[NQ - 1], x[NQ - 1], ss);
            ss = sum_wave(ss);
            float sc = inv_norm_f(ss);
            if (wave == 0) sc = sc * (1.0f / sqrtf((float)DK));
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                act[wave * DK + lane + 64 * j] = x[j] * sc;
#pragma unroll
                for (int k = 0; k < 3; ++k) tl[(size_t)k * C + gq[j]] = xq[j][k + 1];
            }
        }
        if (tid < nv) {
            float y = wv.x * bf16f(xv[0]);
            y = fmaf(wv.y, bf16f(xv[1]), y);
            y = fmaf(wv.z, bf16f(xv[2]), y);
            y = fmaf(wv.w, bf16f(xv[3]), y);
            act[2 * DK + tid] = silu_f(y);
#pragma unroll
            for (int k = 0; k < 3; ++k) tl[(size_t)k * C + gvc] = xv[k + 1];
        }
        if (tid < vpw) {
            galpha[tid] = decay_f(log_decay(av, al, db));
            gbeta[tid] = sigmoid_f(bv);
        }
        lds_barrier();
    }
    if (!row_wave) return;
    wait_vmem();
    const float *qrow = act + grp * R;
    const float *krow = act + DK + grp * R;
    const float4 vv = *reinterpret_cast<const float4 *>(act + 2 * DK + jl * A.dv + col);
    float *dst = A.state_out + ((size_t)s * A.hv + h) * head_elems + lane_off;
    float4 d, o;
    row_step<R, true, false>(m, krow, qrow, vv, galpha[jl], gbeta[jl], dst, A.dv, d, o);
    if (grp == 0) *reinterpret_cast<float4 *>(A.out + ((size_t)s * A.hv + h) * A.dv + col) = o;
}

// Commit: the accepted row's recorded state and tail replace the stream's.
// A row outside the stream's own window (or a window past the recorded rows)
// skips the stream.
__global__ void __launch_bounds__(256) commit_kernel(const CommitArgs A)
{
    const int s = blockIdx.y;
    const int acc = A.accept[s];
    if (acc < 0) return;
    const int r0 = A.row_start[s], r1 = A.row_start[s + 1];
    if (r0 < 0 || r1 > A.total_rows || acc < r0 || acc >= r1) return;
    const size_t nthr = (size_t)gridDim.x * blockDim.x;
    const size_t first = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const float4 *src = reinterpret_cast<const float4 *>(A.state_snap + (size_t)acc * A.state_elems);
    float4 *dst = reinterpret_cast<float4 *>(A.state + (size_t)s * A.state_elems);
    for (size_t i = first; i < A.state_elems / 4; i += nthr) dst[i] = src[i];
    const uint4 *tsrc = reinterpret_cast<const uint4 *>(A.tail_snap + (size_t)acc * A.tail_elems);
    uint4 *tdst = reinterpret_cast<uint4 *>(A.tail + (size_t)s * A.tail_elems);
    for (size_t i = first; i < A.tail_elems / 8; i += nthr) tdst[i] = tsrc[i];
}

// Commit by replay: the kept path of each stream (its accepted row and that
// row's ancestors, root first) is replayed onto the stream's state from the
// log, and the path's last three raw rows (continuing into the old tail)
// become its conv tail.  One workgroup per (stream, value head); thread
// (c4, rg) keeps state rows [rg*RPT, rg*RPT + RPT) x columns [4 c4, 4 c4 + 4)
// in registers while the path's rows go by, reading each row's decay, write
// and key from LDS.  Each state element takes the path's rows in order with
// the row kernel's operations, so the result is the recorded state of the
// accepted row, bit for bit.  The workgroups of a stream share the tail's
// channel groups out.
template <int DK, int DV>
__global__ void __launch_bounds__(256) replay_kernel(const ReplayArgs A)
{
    constexpr int C4 = DV / 4;              // column groups of 4
    constexpr int RPT = DK * C4 / 256;      // state rows a thread keeps
    __shared__ int path[kMaxWindowRows];
    __shared__ int plen;
    __shared__ float pal[kMaxWindowRows];
    __shared__ __align__(16) float pkey[kMaxWindowRows * DK];
    __shared__ __align__(16) float pdel[kMaxWindowRows * DV];
    const int tid = threadIdx.x;
    const int s = blockIdx.x / A.hv, h = blockIdx.x - s * A.hv;
    const int acc = A.accept[s];
    if (acc < 0) return;
    const int r0 = A.row_start[s], r1 = A.row_start[s + 1];
    if (r0 < 0 || r1 < r0 || r1 > A.total_rows || r1 - r0 > A.max_rows || acc < r0 || acc >= r1) return;
    const int c4 = tid % C4, i0 = (tid / C4) * RPT;
    float4 *st = reinterpret_cast<float4 *>(A.state + ((size_t)s * A.hv + h) * DK * DV);
    float4 m[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) m[r] = st[(i0 + r) * C4 + c4];   // in flight while the path is found
    if (tid == 0) {
        // the path from the kept row up to the root, then reversed; a parent
        // outside [-1, row) refuses the stream
        int n = 0, ok = 1;
        for (int i = acc - r0; i >= 0;) {
            const int p = A.parent ? A.parent[r0 + i] : i - 1;
            if (p < -1 || p >= i || n == kMaxWindowRows) {
                ok = 0;
                break;
            }
            path[n++] = i;
            i = p;
        }
        for (int a = 0, b = n - 1; a < b; ++a, --b) {
            const int t = path[a];
            path[a] = path[b];
            path[b] = t;
        }
        plen = ok ? n : 0;
    }
    __syncthreads();
    const int n = plen;
    if (n == 0) return;
    const int kh = h / (A.hv / A.hk);
    for (int idx = tid; idx < n * (DK / 4); idx += 256) {
        const int q = idx / (DK / 4), i4 = idx - q * (DK / 4);
        reinterpret_cast<float4 *>(pkey)[idx] =
            reinterpret_cast<const float4 *>(A.log_key + ((size_t)(r0 + path[q]) * A.hk + kh) * DK)[i4];
    }
    for (int idx = tid; idx < n * C4; idx += 256) {
        const int q = idx / C4, j4 = idx - q * C4;
        reinterpret_cast<float4 *>(pdel)[idx] =
            reinterpret_cast<const float4 *>(A.log_delta + ((size_t)(r0 + path[q]) * A.hv + h) * DV)[j4];
    }
    if (tid < n) pal[tid] = A.log_alpha[(size_t)(r0 + path[tid]) * A.hv + h];
    __syncthreads();

    for (int q = 0; q < n; ++q) {
        const float a = pal[q];
        const float4 d = reinterpret_cast<const float4 *>(pdel + q * DV)[c4];
        float k[RPT];
#pragma unroll
        for (int r = 0; r < RPT; r += 4) {
            const float4 kv = *reinterpret_cast<const float4 *>(pkey + q * DK + i0 + r);
            k[r] = kv.x; k[r + 1] = kv.y; k[r + 2] = kv.z; k[r + 3] = kv.w;
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            m[r].x = fmaf(k[r], d.x, a * m[r].x);
            m[r].y = fmaf(k[r], d.y, a * m[r].y);
            m[r].z = fmaf(k[r], d.z, a * m[r].z);
            m[r].w = fmaf(k[r], d.w, a * m[r].w);
        }
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) st[(i0 + r) * C4 + c4] = m[r];

    // the tail: new row j is path row n - 3 + j, or old tail row n + j before
    // the path; one thread reads a channel group's three rows before writing
    const int C = A.C, units = C / 8;
    uint16_t *tl = A.tail + (size_t)s * 3 * C;
    const uint16_t *src0 = n >= 3 ? A.qkv + (size_t)(r0 + path[n - 3]) * C : tl + (size_t)n * C;
    const uint16_t *src1 = n >= 2 ? A.qkv + (size_t)(r0 + path[n - 2]) * C : tl + (size_t)(n + 1) * C;
    const uint16_t *src2 = A.qkv + (size_t)(r0 + path[n - 1]) * C;
    for (int u = h * 256 + tid; u < units; u += A.hv * 256) {
        const uint4 x0 = *reinterpret_cast<const uint4 *>(src0 + 8 * u);
        const uint4 x1 = *reinterpret_cast<const uint4 *>(src1 + 8 * u);
        const uint4 x2 = *reinterpret_cast<const uint4 *>(src2 + 8 * u);
        *reinterpret_cast<uint4 *>(tl + 8 * u) = x0;
        *reinterpret_cast<uint4 *>(tl + (size_t)C + 8 * u) = x1;
        *reinterpret_cast<uint4 *>(tl + (size_t)2 * C + 8 * u) = x2;
    }
}

}  // namespace

// The row loop needs 64 * vpw * dv/32/cs threads.  When the launch has no more
// workgroups than the chip has CUs (256), each gets at least 512: the extra
// waves take part in the prologue (staging, conv, norms) and then leave.
int rows_block_threads(const RowsArgs &A)
{
    const long long wgs = (long long)A.n_streams * A.hk * (A.r / A.vpw) * A.cs;
    const int need = 64 * A.vpw * (A.dv / 32 / A.cs);
    return wgs <= 256 ? max(need, 512) : need;
}

// row waves of a workgroup: vpw value heads of dv / 32 / cs column tiles each
static size_t row_waves(const RowsArgs &A) { return (size_t)A.vpw * (A.dv / 32 / A.cs); }

size_t rows_lds_bytes(const RowsArgs &A)
{
    return rows_state_cache_offset(A)
           + (A.mode == MODE_TREE ? sizeof(float) * 4 * 64 * row_waves(A) * A.cache_rows : 0);
}

int rows_cache_rows_that_fit(const RowsArgs &A)
{
    const size_t rows = (size_t)A.dk / 32;   // a quarter of a lane's dk / 8 rows
    const size_t need = rows_state_cache_offset(A) + sizeof(float) * 4 * 64 * row_waves(A) * rows;
    return A.mode == MODE_TREE && need <= kRowsMaxLds ? (int)rows : 0;
}

namespace {
// Dynamic LDS above the 64 KiB default has to be allowed per kernel once.
template <int DK, bool LOG, bool NT>
hipError_t launch_rows_as(const RowsArgs &A, dim3 grid, dim3 block, size_t lds, hipStream_t stream)
{
    static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&rows_kernel<DK, LOG, NT>),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                                    (int)kRowsMaxLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((rows_kernel<DK, LOG, NT>), grid, block, lds, stream, A);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_rows_dk(const RowsArgs &A, dim3 grid, dim3 block, size_t lds, hipStream_t stream)
{
    if (A.logged) return launch_rows_as<DK, true, false>(A, grid, block, lds, stream);
    if (A.mode == MODE_TREE) return launch_rows_as<DK, false, true>(A, grid, block, lds, stream);
    return launch_rows_as<DK, false, false>(A, grid, block, lds, stream);
}
}  // namespace

hipError_t launch_step(const RowsArgs &A, hipStream_t stream)
{
    const dim3 grid((unsigned)A.n_streams, (unsigned)A.hk);
    const dim3 block(max(128, 64 * A.r * (A.dv / 32)));
    const size_t lds = sizeof(float) * (2 * (size_t)A.dk + (size_t)A.r * A.dv + 2 * (size_t)A.r);
    if (A.dk == 128)
        hipLaunchKernelGGL((step_kernel<128>), grid, block, lds, stream, A);
    else
        hipLaunchKernelGGL((step_kernel<64>), grid, block, lds, stream, A);
    return hipGetLastError();
}

hipError_t launch_rows(const RowsArgs &A, hipStream_t stream)
{
    const dim3 grid((unsigned)A.n_streams * A.hk * (A.r / A.vpw) * A.cs);
    const dim3 block(rows_block_threads(A));
    const size_t lds = rows_lds_bytes(A);
    if (lds > kRowsMaxLds) return hipErrorInvalidValue;
    return A.dk == 128 ? launch_rows_dk<128>(A, grid, block, lds, stream)
                       : launch_rows_dk<64>(A, grid, block, lds, stream);
}

hipError_t launch_commit(const CommitArgs &A, hipStream_t stream)
{
    const dim3 grid(48, (unsigned)A.n_streams);
    hipLaunchKernelGGL(commit_kernel, grid, dim3(256), 0, stream, A);
    return hipGetLastError();
}

hipError_t launch_replay(const ReplayArgs &A, hipStream_t stream)
{
    const dim3 grid((unsigned)A.n_streams * A.hv);
    if (A.dk == 128 && A.dv == 128)
        hipLaunchKernelGGL((replay_kernel<128, 128>), grid, dim3(256), 0, stream, A);
    else if (A.dk == 128)
        hipLaunchKernelGGL((replay_kernel<128, 64>), grid, dim3(256), 0, stream, A);
    else if (A.dv == 128)
        hipLaunchKernelGGL((replay_kernel<64, 128>), grid, dim3(256), 0, stream, A);
    else
        hipLaunchKernelGGL((replay_kernel<64, 64>), grid, dim3(256), 0, stream, A);
    return hipGetLastError();
}

}  // namespace gdn
