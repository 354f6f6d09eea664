// Row kernels of libgdn: one-row steps, verify windows and verify trees of the
// gated-delta-rule mixer, plus the commit copy.  gfx950 (CDNA4), wave64.
//
// One workgroup serves one stream and `vpw` value heads of one key head.
//
//   prologue  every (row, channel) of the window: causal conv (taps along the
//             row's own branch) + SiLU into LDS; gates per (row, value head);
//             then per row an L2 norm of q and of k (q also times dk^-1/2).
//             Raw tail rows are copied to the tail snapshots here.
//   rows      each wave owns 64 columns of one value head's state M = S^T
//             ([dk][dv], dv contiguous).  Lane (c, g) = (lane & 15, lane >> 4)
//             keeps rows [g*dk/4, (g+1)*dk/4) x columns [4c, 4c+4) of the
//             tile in VGPRs for the whole window, so the state crosses HBM
//             once on the way in; the per-row snapshot is written with
//             dwordx4 stores that form full 256-byte row segments.
//             The two dk-sums (M^T k and M^T q) are per-lane partials over the
//             lane's rows, then a butterfly over the four 16-lane rows with the
//             gfx950 lane-swap instructions.  No barrier inside the row loop,
//             and no global load except a tree row's parent-state reload.
//
// Every row of every mode runs this same code in the same order, so a window's
// rows equal one-row steps bit for bit and a tree's paths equal chains (the
// pages require window rows to equal one-row steps bit for bit: page
// "perf(qwen3_5 cuda): deliver the first token before drafting", commit note
// on the MLX affine 4-bit checkpoint).  The build disables fp contraction;
// every fused multiply-add below is written out.
#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __forceinline__ float bf16f(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }

// softplus(x) = log(1 + e^x) without overflow or cancellation.
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }

__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

__device__ __forceinline__ float silu_f(float y) { return y / (1.0f + expf(-y)); }

// Sum over the four 16-lane rows of the wave; every lane gets the same bits.
// permlane16_swap pairs rows (0,1) and (2,3), permlane32_swap the two halves.
__device__ __forceinline__ float sum_rows4(float x)
{
    const uint32_t xi = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
    const float s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const uint32_t si = __float_as_uint(s);
    const auto q = __builtin_amdgcn_permlane32_swap(si, si, false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Sum over all 64 lanes (butterfly, the same bits in every lane).
__device__ __forceinline__ float sum_wave(float x)
{
    x = x + __shfl_xor(x, 1);
    x = x + __shfl_xor(x, 2);
    x = x + __shfl_xor(x, 4);
    x = x + __shfl_xor(x, 8);
    return sum_rows4(x);
}

// Global channel of local prologue channel `ch`: [q of kh | k of kh | v of
// the workgroup's value heads].
__device__ __forceinline__ int global_channel(const RowsArgs &A, int dk, int kh, int h0, int ch)
{
    if (ch < dk) return kh * dk + ch;
    if (ch < 2 * dk) return A.hk * dk + kh * dk + (ch - dk);
    return 2 * A.hk * dk + h0 * A.dv + (ch - 2 * dk);
}

template <int DK>
__global__ void __launch_bounds__(512) rows_kernel(const RowsArgs A)
{
    constexpr int R = DK / 4;  // state rows held by one lane
    extern __shared__ float smem[];

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int groups = A.r / A.vpw;
    int bid = blockIdx.x;
    const int g = bid % groups;
    bid /= groups;
    const int kh = bid % A.hk;
    const int s = bid / A.hk;
    const int h0 = kh * A.r + g * A.vpw;   // first value head of this workgroup

    // ---- layout of this stream's rows (device-side rules; a stream that
    // breaks them is skipped)
    int r0, r1;
    if (A.mode == MODE_STEP) {
        r0 = s;
        r1 = s + 1;
    } else {
        r0 = A.row_start[s];
        r1 = A.row_start[s + 1];
    }
    if (r0 < 0 || r1 < r0 || r1 > A.total_rows || r1 - r0 > A.max_rows) return;
    const int len = r1 - r0;
    if (len == 0) return;

    const int nch = 2 * DK + A.vpw * A.dv;
    float *act = smem;                                 // [max_rows][nch]
    float *galpha = act + A.max_rows * nch;            // [max_rows][vpw]
    float *gbeta = galpha + A.max_rows * A.vpw;        // [max_rows][vpw]
    int *anc = reinterpret_cast<int *>(gbeta + A.max_rows * A.vpw);  // [max_rows][4]
    int *bad = anc + A.max_rows * 4;

    // ---- this wave's tile of the state: issue its loads first
    const int waves_per_head = A.dv / 64;
    const int jl = wave / waves_per_head;       // local value head
    const int tile = wave - jl * waves_per_head;
    const int h = h0 + jl;
    const int c4 = lane & 15, grp = lane >> 4;
    const int col = tile * 64 + c4 * 4;
    const size_t head_elems = (size_t)DK * A.dv;
    const size_t lane_off = (size_t)(grp * R) * A.dv + col;
    const float *st_in = A.state_in + ((size_t)s * A.hv + h) * head_elems + lane_off;
    float4 m[R];
#pragma unroll
    for (int i = 0; i < R; ++i) m[i] = *reinterpret_cast<const float4 *>(st_in + (size_t)i * A.dv);

    // ---- parents and the three nearest ancestors of every row.  anc[t][0]
    // is the parent (whose state row t starts from); anc[t][d] is the source
    // of x_{t-d}: a local row >= 0, or -1, -2, -3 for tail rows 2, 1, 0.
    if (tid == 0) *bad = 0;
    if (tid < len) anc[tid * 4] = (A.mode == MODE_TREE) ? A.parent[r0 + tid] : tid - 1;
    __syncthreads();
    if (tid < len && (anc[tid * 4] < -1 || anc[tid * 4] >= tid)) *bad = 1;
    __syncthreads();
    if (*bad) return;
    if (tid < len) {
        int i = tid;
#pragma unroll
        for (int d = 1; d <= 3; ++d) {
            i = (i >= 0) ? anc[i * 4] : i - 1;
            anc[tid * 4 + d] = i;
        }
    }
    __syncthreads();

    // ---- conv + SiLU of every (row, channel); tail snapshots
    const int C = A.C;
    const uint16_t *tail = A.tail_in + (size_t)s * 3 * C;
    const uint16_t *rows = A.qkv + (size_t)r0 * C;
    const bool record = (A.mode != MODE_STEP);
    for (int idx = tid; idx < len * nch; idx += nthr) {
        const int t = idx / nch;
        const int ch = idx - t * nch;
        const int gc = global_channel(A, DK, kh, h0, ch);
        const int a1 = anc[t * 4 + 1], a2 = anc[t * 4 + 2], a3 = anc[t * 4 + 3];
        const uint16_t x3 = rows[(size_t)t * C + gc];
        const uint16_t x2 = a1 >= 0 ? rows[(size_t)a1 * C + gc] : tail[(3 + a1) * C + gc];
        const uint16_t x1 = a2 >= 0 ? rows[(size_t)a2 * C + gc] : tail[(3 + a2) * C + gc];
        const uint16_t x0 = a3 >= 0 ? rows[(size_t)a3 * C + gc] : tail[(3 + a3) * C + gc];
        const float4 w = *reinterpret_cast<const float4 *>(A.conv_w + (size_t)gc * 4);
        float y = w.x * bf16f(x0);
        y = fmaf(w.y, bf16f(x1), y);
        y = fmaf(w.z, bf16f(x2), y);
        y = fmaf(w.w, bf16f(x3), y);
        act[t * nch + ch] = silu_f(y);
        // q/k channels are shared by the key head's workgroups: group 0 records them
        if (record && (ch >= 2 * DK || g == 0)) {
            uint16_t *ts = A.tail_snap + (size_t)(r0 + t) * 3 * C + gc;
            ts[0] = x1;
            ts[C] = x2;
            ts[2 * C] = x3;
        }
    }
    // ---- gates of every (row, value head)
    for (int idx = tid; idx < len * A.vpw; idx += nthr) {
        const int t = idx / A.vpw;
        const int j = idx - t * A.vpw;
        const int hh = h0 + j;
        const float av = bf16f(A.a[(size_t)(r0 + t) * A.hv + hh]);
        const float bv = bf16f(A.b[(size_t)(r0 + t) * A.hv + hh]);
        const float gl = -expf(A.a_log[hh]) * softplus_f(av + A.dt_bias[hh]);
        galpha[t * A.vpw + j] = expf(gl);
        gbeta[t * A.vpw + j] = sigmoid_f(bv);
    }
    __syncthreads();

    // ---- one-row step: the new tail replaces the old one in place.  All of
    // this workgroup's tail reads are behind the barrier above, and (with one
    // workgroup per key head in this mode) no other workgroup reads these
    // channels.
    if (A.mode == MODE_STEP) {
        uint16_t *tl = A.tail_out + (size_t)s * 3 * C;
        for (int ch = tid; ch < nch; ch += nthr) {
            const int gc = global_channel(A, DK, kh, h0, ch);
            const uint16_t t1 = tl[C + gc], t2 = tl[2 * C + gc];
            tl[gc] = t1;
            tl[C + gc] = t2;
            tl[2 * C + gc] = rows[gc];
        }
    }

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
            float sc = 1.0f / sqrtf(ss + 1e-6f);
            if (which == 0) sc = sc * qscale;
            v[lane] = x0 * sc;
            if (DK == 128) v[lane + 64] = x1 * sc;
        }
    }
    __syncthreads();

    // ---- the recurrence, row after row, on the tile held in registers
    const float *st_in_head = A.state_in + ((size_t)s * A.hv + h) * head_elems + lane_off;
    int prev = -1;
    for (int t = 0; t < len; ++t) {
        const int p = anc[t * 4];
        if (p != prev) {
            // a tree row whose parent is not the row just done: reload the
            // parent's state (the stream's own state for p == -1).  These
            // are the addresses this lane itself stored.
            const float *src = p < 0 ? st_in_head
                                     : A.state_snap + ((size_t)(r0 + p) * A.hv + h) * head_elems + lane_off;
#pragma unroll
            for (int i = 0; i < R; ++i) m[i] = *reinterpret_cast<const float4 *>(src + (size_t)i * A.dv);
        }
        const float *qrow = act + t * nch + grp * R;
        const float *krow = act + t * nch + DK + grp * R;

        // u = M^T k (over the lane's rows, then across the four row groups)
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
        u.x = sum_rows4(u.x);
        u.y = sum_rows4(u.y);
        u.z = sum_rows4(u.z);
        u.w = sum_rows4(u.w);

        // delta = beta (v - alpha u);  M <- alpha M + k delta^T;  o = M^T q
        const float al = galpha[t * A.vpw + jl];
        const float be = gbeta[t * A.vpw + jl];
        const float4 vv = *reinterpret_cast<const float4 *>(act + t * nch + 2 * DK + jl * A.dv + col);
        float4 d;
        d.x = be * (vv.x - al * u.x);
        d.y = be * (vv.y - al * u.y);
        d.z = be * (vv.z - al * u.z);
        d.w = be * (vv.w - al * u.w);
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
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
            }
        }
        o.x = sum_rows4(o.x);
        o.y = sum_rows4(o.y);
        o.z = sum_rows4(o.z);
        o.w = sum_rows4(o.w);

        const int row = r0 + t;
        if (grp == 0)
            *reinterpret_cast<float4 *>(A.out + ((size_t)row * A.hv + h) * A.dv + col) = o;
        float *dst = (A.mode == MODE_STEP)
                         ? A.state_out + ((size_t)s * A.hv + h) * head_elems + lane_off
                         : A.state_snap + ((size_t)row * A.hv + h) * head_elems + lane_off;
#pragma unroll
        for (int i = 0; i < R; ++i) *reinterpret_cast<float4 *>(dst + (size_t)i * A.dv) = m[i];
        prev = t;
    }
}

// Commit: the accepted row's recorded state and tail replace the stream's.
__global__ void __launch_bounds__(256) commit_kernel(const CommitArgs A)
{
    const int s = blockIdx.y;
    const int acc = A.accept[s];
    if (acc < 0 || acc >= A.total_rows) return;
    const size_t nthr = (size_t)gridDim.x * blockDim.x;
    const size_t first = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const float4 *src = reinterpret_cast<const float4 *>(A.state_snap + (size_t)acc * A.state_elems);
    float4 *dst = reinterpret_cast<float4 *>(A.state + (size_t)s * A.state_elems);
    for (size_t i = first; i < A.state_elems / 4; i += nthr) dst[i] = src[i];
    const uint4 *tsrc = reinterpret_cast<const uint4 *>(A.tail_snap + (size_t)acc * A.tail_elems);
    uint4 *tdst = reinterpret_cast<uint4 *>(A.tail + (size_t)s * A.tail_elems);
    for (size_t i = first; i < A.tail_elems / 8; i += nthr) tdst[i] = tsrc[i];
}

}  // namespace

int rows_block_threads(const RowsArgs &A) { return 64 * A.vpw * (A.dv / 64); }

size_t rows_lds_bytes(const RowsArgs &A)
{
    const size_t nch = 2 * (size_t)A.dk + (size_t)A.vpw * A.dv;
    return sizeof(float) * ((size_t)A.max_rows * nch + 2 * (size_t)A.max_rows * A.vpw) +
           sizeof(int) * (4 * (size_t)A.max_rows + 1);
}

hipError_t launch_rows(const RowsArgs &A, hipStream_t stream)
{
    const dim3 grid((unsigned)A.n_streams * A.hk * (A.r / A.vpw));
    const dim3 block(rows_block_threads(A));
    const size_t lds = rows_lds_bytes(A);
    if (A.dk == 128)
        hipLaunchKernelGGL(rows_kernel<128>, grid, block, lds, stream, A);
    else
        hipLaunchKernelGGL(rows_kernel<64>, grid, block, lds, stream, A);
    return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs &A, hipStream_t stream)
{
    const dim3 grid(48, (unsigned)A.n_streams);
    hipLaunchKernelGGL(commit_kernel, grid, dim3(256), 0, stream, A);
    return hipGetLastError();
}

}  // namespace gdn
