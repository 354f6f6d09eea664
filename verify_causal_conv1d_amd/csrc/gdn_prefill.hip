// Chunked prompt pass of libgdn (gfx950): the gated delta rule in chunkwise
// WY form, chunks of 64 rows that never cross prompts.
//
// Within a chunk that starts from state M0 (M = S^T, [dk][dv]), with
// g_t = log alpha_t and gamma_t = g_1 + ... + g_t (in-chunk),
//   A_tj = beta_t e^{gamma_t - gamma_j} k_t.k_j (j < t),  T = (I + A)^-1,
//   W = T (beta e^gamma k),  U~ = T (beta v),  U = U~ - W M0,
//   O = (e^gamma q) M0 + P U,  P_tj = e^{gamma_t - gamma_j} q_t.k_j (j <= t),
//   M_next = e^{gamma_L} M0 + (e^{gamma_L - gamma} k)^T U.
// (The derivation unrolls M_t = alpha_t M_{t-1} + k_t d_t^T with
// d_t = beta_t (v_t - alpha_t M_{t-1}^T k_t) over the chunk; the gated delta
// rule is Yang, Kautz and Hatamizadeh, "Gated Delta Networks", 2024.)
//
// Three launches on the caller's stream:
//   prologue  per 32 packed rows x key head: causal conv (taps from the
//             prompt's own earlier rows or its tail) + SiLU, q/k L2 norms,
//             gates.  q^, k^, v are stored as bf16 (the matrix-core operand
//             type), log alpha and beta as fp32.
//   intra     per (chunk, key head): K K^T and Q K^T on bf16 MFMA
//             (v_mfma_f32_32x32x16_bf16); per value head gamma, the fp32
//             triangular solve for T (one wave, one column a lane), and W^T,
//             U~ on bf16 MFMA.  Everything the sweep needs leaves this kernel
//             in the exact lane order of the sweep's MFMA operands, so the
//             sweep reads each operand with two 16-byte loads a lane.
//   sweep     per (prompt, value head, 32 state columns), 4 waves, each
//             holding 32 rows of the state as an fp32 MFMA accumulator: the
//             state contractions U~ - W M0, (e^gamma q) M0, P U and the update
//             (e^{gamma_L - gamma} k)^T U run on fp32 MFMA
//             (v_mfma_f32_32x32x2_f32) with the accumulator itself as the B
//             operand; partial sums over the four row blocks meet in LDS.
//             Sequential over the prompt's chunks, with each operand of chunk
//             c + 1 fetched right after its last use in chunk c; the state
//             never leaves the chip between chunks.  Workgroups take prompts
//             longest first, so the longest dependency chain starts first.
// The prompt's final state replaces the stream's state and its last three raw
// rows (or a mix with the old tail for prompts shorter than three rows) its
// conv tail, in place (prompt passes update the stream in place: page
// "perf(qwen3_5 cuda): deliver the first token before drafting", commit note
// on tree-shaped verify windows).
#include "gdn_device.h"
#include "gdn_prefill.h"

namespace gdn {
namespace {

constexpr int DKP = 128;        // head sizes this pass is built for
constexpr int PRO_ROWS = 32;    // packed rows a prologue workgroup
constexpr int TILE = 32;        // state columns a sweep workgroup
constexpr int HB = 3;           // value heads whose triangular solves run side by side

// A chunk-head block of sweep operands (bf16), every sub-array in lane order
// [.][.][64 lanes][16], lane l = (l32, hh) = (l & 31, l >> 5):
//   W  [mb][w]     lane value i = W[32 mb + l32][32 w + kx(i)]
//   QE [mb][w]     lane value i = e^{gamma_t} q^[t = 32 mb + l32][32 w + kx(i)]
//   KT [mb][w]     lane value i = e^{gamma_L - gamma_t} k^[t = 32 mb + kx(i)][32 w + l32]
//   P  [mb][mbk]   lane value i = P[32 mb + l32][32 mbk + kx(i)]
//   UT [mb][tile]  lane value i = U~[32 mb + kx(i)][32 tile + l32]
// with kx(i) = 8 (i / 4) + 4 hh + i % 4: the k index that lane l feeds at step
// i of a v_mfma_f32_32x32x2_f32 chain whose B operand is register i of a
// 32 x 32 accumulator (accumulator register i of lane l holds row kx(i),
// column l32).  Rows past the chunk's end are zero.
constexpr int kOffW = 0, kOffQE = 8192, kOffKT = 16384, kOffP = 24576, kOffUT = 28672;
constexpr int kBlockElems = 36864;

struct Ctx {
    PrefillArgs P;
    int r;                      // value heads per key head
    int max_chunks;             // chunks of the longest prompt (bounds the intra grid)
    int nc_total;               // chunk blocks in the workspace
    uint16_t *qk, *v, *blk;
    float *g, *be, *el;
};

__device__ __forceinline__ int kx(int i, int hh) { return 8 * (i >> 2) + 4 * hh + (i & 3); }

// Rows of prompt p, and the dense index of its first chunk.  False if p or an
// earlier prompt breaks the layout rules (monotone starts within [0, T],
// lengths <= max_len); such a prompt is skipped.
__device__ bool prompt_chunks(const Ctx &X, int p, int &s0, int &s1, int &cid0)
{
    const int T = X.P.total_rows;
    int base = 0;
    int prev = X.P.seq_start[0];
    if (prev < 0) return false;
    for (int q = 0; q <= p; ++q) {
        const int a = X.P.seq_start[q], b = X.P.seq_start[q + 1];
        if (a != prev || b < a || b > T || b - a > X.P.max_len) return false;
        prev = b;
        if (q < p) base += (b - a + kChunk - 1) / kChunk;
    }
    s0 = X.P.seq_start[p];
    s1 = X.P.seq_start[p + 1];
    cid0 = base;
    return base + (s1 - s0 + kChunk - 1) / kChunk <= X.nc_total;
}

// Local prologue channel -> global channel: [q of kh | k of kh | v of kh's value heads].
__device__ __forceinline__ int pro_channel(const Ctx &X, int kh, int ch)
{
    if (ch < DKP) return kh * DKP + ch;
    if (ch < 2 * DKP) return X.P.hk * DKP + kh * DKP + (ch - DKP);
    return 2 * X.P.hk * DKP + kh * X.r * DKP + (ch - 2 * DKP);
}

// ---------------------------------------------------------------- prologue
__global__ void __launch_bounds__(256) prologue_kernel(const Ctx X)
{
    extern __shared__ float smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kh = blockIdx.y;
    const int t0 = blockIdx.x * PRO_ROWS;
    const int T = X.P.total_rows;
    const int nrows = min(PRO_ROWS, T - t0);
    const int C = X.P.C;
    const int nch = 2 * DKP + X.r * DKP;
    float *act = smem;                                                    // [PRO_ROWS][2*DKP]
    float4 *wl = reinterpret_cast<float4 *>(act + PRO_ROWS * 2 * DKP);    // [nch]
    uint16_t *raw = reinterpret_cast<uint16_t *>(wl + nch);               // [PRO_ROWS + 3][nch]
    int *rstart = reinterpret_cast<int *>(raw + (PRO_ROWS + 3) * nch);    // [PRO_ROWS]
    int *rprompt = rstart + PRO_ROWS;                                     // [PRO_ROWS]

    // prompt of each row: the last p with seq_start[p] <= t, if t < seq_start[p + 1]
    if (tid < nrows) {
        const int t = t0 + tid;
        int lo = 0, hi = X.P.n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (X.P.seq_start[mid] <= t) lo = mid; else hi = mid - 1;
        }
        const int s0 = X.P.seq_start[lo], s1 = X.P.seq_start[lo + 1];
        const bool ok = s0 >= 0 && s0 <= t && t < s1 && s1 <= T && s1 - s0 <= X.P.max_len;
        rstart[tid] = ok ? s0 : -1;
        rprompt[tid] = lo;
    }
    // stage raw rows t0-3 .. t0+nrows-1 of this key head's channels, and the weights
    {
        const int cpr = nch / 8;
        const int nchunks = (nrows + 3) * cpr;
        constexpr int B = 8;
        for (int base = 0; base < nchunks; base += B * 256) {
            uint4 v[B];
#pragma unroll
            for (int k = 0; k < B; ++k) {
                const int idx = base + k * 256 + tid;
                const int j = idx / cpr;
                const int u = t0 - 3 + j;
                if (idx < nchunks && u >= 0)
                    v[k] = *reinterpret_cast<const uint4 *>(X.P.qkv + (size_t)u * C +
                                                            pro_channel(X, kh, (idx - j * cpr) * 8));
            }
#pragma unroll
            for (int k = 0; k < B; ++k) {
                const int idx = base + k * 256 + tid;
                const int j = idx / cpr;
                if (idx < nchunks && t0 - 3 + j >= 0)
                    *reinterpret_cast<uint4 *>(raw + j * nch + (idx - j * cpr) * 8) = v[k];
            }
        }
        for (int ch = tid; ch < nch; ch += 256)
            wl[ch] = *reinterpret_cast<const float4 *>(X.P.conv_w + (size_t)pro_channel(X, kh, ch) * 4);
    }
    lds_barrier();

    // gates of every (row, value head of kh)
    for (int idx = tid; idx < nrows * X.r; idx += 256) {
        const int i = idx / X.r;
        if (rstart[i] < 0) continue;
        const int h = kh * X.r + (idx - i * X.r);
        const size_t o = (size_t)(t0 + i) * X.P.hv + h;
        X.g[o] = log_decay(bf16f(X.P.a[o]), X.P.a_log[h], X.P.dt_bias[h]);
        X.be[o] = sigmoid_f(bf16f(X.P.b[o]));
    }
    // conv + SiLU, a thread walking the rows of one channel: q/k into LDS for
    // the norms, v straight out as bf16
    for (int ch = tid; ch < nch; ch += 256) {
        const float4 w = wl[ch];
        const int gc = pro_channel(X, kh, ch);
        for (int i = 0; i < nrows; ++i) {
            const int rs = rstart[i];
            if (rs < 0) continue;
            const int t = t0 + i;
            // tap j reads x_{t-3+j}: a staged row of this prompt, or its tail
            const uint16_t *tailc = X.P.conv_tail + (size_t)rprompt[i] * 3 * C + gc;
            const float x0 = bf16f(t - 3 >= rs ? raw[i * nch + ch] : tailc[(size_t)(t - rs) * C]);
            const float x1 = bf16f(t - 2 >= rs ? raw[(i + 1) * nch + ch] : tailc[(size_t)(1 + t - rs) * C]);
            const float x2 = bf16f(t - 1 >= rs ? raw[(i + 2) * nch + ch] : tailc[(size_t)(2 + t - rs) * C]);
            const float x3 = bf16f(raw[(i + 3) * nch + ch]);
            float y = w.x * x0;
            y = fmaf(w.y, x1, y);
            y = fmaf(w.z, x2, y);
            y = fmaf(w.w, x3, y);
            const float a = silu_f(y);
            if (ch < 2 * DKP)
                act[i * 2 * DKP + ch] = a;
            else
                X.v[(size_t)t * X.P.hv * DKP + (size_t)kh * X.r * DKP + (ch - 2 * DKP)] = f2bf(a);
        }
    }
    lds_barrier();

    // L2 norms of q (times dk^-1/2) and k, one wave a (row, q|k) pair
    const float qscale = 1.0f / sqrtf((float)DKP);
    for (int pr = wave; pr < 2 * nrows; pr += 4) {
        const int i = pr >> 1, which = pr & 1;
        if (rstart[i] < 0) continue;
        const float *src = act + i * 2 * DKP + which * DKP;
        const float x0 = src[lane], x1 = src[lane + 64];
        float ss = x0 * x0;
        ss = fmaf(x1, x1, ss);
        ss = sum_wave(ss);
        float sc = 1.0f / sqrtf(ss + 1e-6f);
        if (which == 0) sc = sc * qscale;
        uint16_t *dst = X.qk + ((size_t)(t0 + i) * X.P.hk + kh) * 2 * DKP + which * DKP;
        dst[lane] = f2bf(x0 * sc);
        dst[lane + 64] = f2bf(x1 * sc);
    }
}

// ---------------------------------------------------------------- intra
__device__ __forceinline__ bf8v lds8(const uint16_t *p) { return __builtin_bit_cast(bf8v, *reinterpret_cast<const uint4 *>(p)); }

// Row T_ of the forward substitution T (I + A) = I for unit lower-triangular
// I + A: lane c keeps column c of T; An holds -A (row-major, [64][64]).
template <int T_>
__device__ __forceinline__ void tsolve_row(float (&Tc)[64], const float *An, int lane)
{
    float acc = (T_ == lane) ? 1.0f : 0.0f;
    const float *row = An + T_ * 64;
#pragma unroll
    for (int s4 = 0; s4 + 4 <= T_; s4 += 4) {
        const float4 a4 = *reinterpret_cast<const float4 *>(row + s4);
        acc = fmaf(a4.x, Tc[s4], acc);
        acc = fmaf(a4.y, Tc[s4 + 1], acc);
        acc = fmaf(a4.z, Tc[s4 + 2], acc);
        acc = fmaf(a4.w, Tc[s4 + 3], acc);
    }
#pragma unroll
    for (int s = T_ & ~3; s < T_; ++s) acc = fmaf(row[s], Tc[s], acc);
    Tc[T_] = acc;
    // keep the scheduler from hoisting later rows' LDS reads above this one
    // (it would hold hundreds of them in registers)
    __builtin_amdgcn_sched_barrier(0);
}

template <int T_>
__device__ __forceinline__ void tsolve(float (&Tc)[64], const float *An, int lane)
{
    tsolve_row<T_>(Tc, An, lane);
    if constexpr (T_ + 1 < 64) tsolve<T_ + 1>(Tc, An, lane);
}

__device__ __forceinline__ void store16(uint16_t *dst, const float (&v)[16])
{
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (uint32_t)f2bf(v[2 * e]) | ((uint32_t)f2bf(v[2 * e + 1]) << 16);
    reinterpret_cast<uint4 *>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    reinterpret_cast<uint4 *>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

__global__ void __launch_bounds__(256) intra_kernel(const Ctx X)
{
    extern __shared__ float smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int kh = blockIdx.y;
    const int pidx = blockIdx.x / X.max_chunks, c = blockIdx.x - pidx * X.max_chunks;
    int s0, s1, cid0;
    if (!prompt_chunks(X, pidx, s0, s1, cid0)) return;
    const int r0 = s0 + c * kChunk;
    if (r0 >= s1) return;
    const int L = min(kChunk, s1 - r0);
    const int hv = X.P.hv, hk = X.P.hk;

    uint16_t *qkr = reinterpret_cast<uint16_t *>(smem);            // [64][256] q^ | k^ rows
    float *Skk = reinterpret_cast<float *>(qkr + 64 * 2 * DKP);    // [64][64]
    float *Sqk = Skk + 64 * 64;                                    // [64][64]
    float *An = Sqk + 64 * 64;                                     // [HB][64][64] -A, later KbT / VbT
    uint16_t *Tb = reinterpret_cast<uint16_t *>(An + HB * 64 * 64);   // [HB][64][64] bf16
    float *gam = reinterpret_cast<float *>(Tb + HB * 64 * 64);       // [HB][64]
    float *bet = gam + HB * 64;                                        // [HB][64]
    uint16_t *KbT = reinterpret_cast<uint16_t *>(An);                  // [128][64]
    uint16_t *VbT = KbT + 128 * 64;                                    // [128][64]

    // the chunk's q^ | k^ rows (zero past its end)
    for (int idx = tid; idx < 64 * 32; idx += 256) {
        const int t = idx >> 5, q8 = (idx & 31) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t < L) v = *reinterpret_cast<const uint4 *>(X.qk + ((size_t)(r0 + t) * hk + kh) * 2 * DKP + q8);
        *reinterpret_cast<uint4 *>(qkr + t * 2 * DKP + q8) = v;
    }
    lds_barrier();

    // K K^T and Q K^T: wave w computes the 32 x 32 block (w >> 1, w & 1) of both
    {
        const int bi = wave >> 1, bj = wave & 1;
        const uint16_t *ra = qkr + (32 * bi + l32) * 2 * DKP;
        const uint16_t *rb = qkr + (32 * bj + l32) * 2 * DKP + DKP;
        f16v kk = {}, qk = {};
#pragma unroll
        for (int ks = 0; ks < DKP / 16; ++ks) {
            const int ko = 16 * ks + 8 * hh;
            const bf8v bk = lds8(rb + ko);
            kk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(ra + DKP + ko), bk, kk, 0, 0, 0);
            qk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(ra + ko), bk, qk, 0, 0, 0);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 32 * bi + kx(rr, hh);
            Skk[row * 64 + 32 * bj + l32] = kk[rr];
            Sqk[row * 64 + 32 * bj + l32] = qk[rr];
        }
    }

    for (int j0 = 0; j0 < X.r; j0 += HB) {
        const int nh = min(HB, X.r - j0);
        // gamma (inclusive in-chunk scan of log alpha) and beta, one wave a head
        if (wave < nh) {
            const int h = kh * X.r + j0 + wave;
            const size_t o = (size_t)(r0 + lane) * hv + h;
            float gl = lane < L ? X.g[o] : 0.0f;
            const float bl = lane < L ? X.be[o] : 0.0f;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float up = __shfl_up(gl, d);
                if (lane >= d) gl += up;
            }
            gam[wave * 64 + lane] = gl;
            bet[wave * 64 + lane] = bl;
        }
        lds_barrier();

        if (wave < nh) {
            // -A, column `lane`: -beta_t e^{gamma_t - gamma_s} (k_t . k_s) for t > s
            const float *gj = gam + wave * 64, *bj = bet + wave * 64;
            float *Aj = An + wave * 64 * 64;
            const int s = lane;
            const float gs = gj[s];
            for (int t = 0; t < 64; ++t)
                Aj[t * 64 + s] = t > s ? -bj[t] * __expf(gj[t] - gs) * Skk[t * 64 + s] : 0.0f;
            // T = (I + A)^-1 by forward substitution; lane c keeps column c
            float Tc[64];
            tsolve<0>(Tc, Aj, lane);
            uint16_t *Tj = Tb + wave * 64 * 64;
#pragma unroll
            for (int t = 0; t < 64; ++t) Tj[t * 64 + lane] = f2bf(Tc[t]);
        }
        lds_barrier();

        for (int jj = 0; jj < nh; ++jj) {
            const int h = kh * X.r + j0 + jj;
            const float *gj = gam + jj * 64, *bj = bet + jj * 64;
            const float gL = gj[63];
            uint16_t *blk = X.blk + ((size_t)(cid0 + c) * hv + h) * kBlockElems;
            // KbT[k][s] = beta_s e^{gamma_s} k_s[k],  VbT[c][s] = beta_s v_s[c]
            for (int idx = tid; idx < 64 * 16 * 2; idx += 256) {
                const int which = idx >= 64 * 16;
                const int id = idx - which * 64 * 16;
                const int s = id >> 4, q8 = (id & 15) * 8;
                uint4 raw = make_uint4(0, 0, 0, 0);
                if (which && s < L) raw = *reinterpret_cast<const uint4 *>(X.v + ((size_t)(r0 + s) * hv + h) * DKP + q8);
                if (!which) raw = *reinterpret_cast<const uint4 *>(qkr + s * 2 * DKP + DKP + q8);
                const uint16_t *e8 = reinterpret_cast<const uint16_t *>(&raw);
                const float sc = which ? bj[s] : bj[s] * __expf(gj[s]);
                uint16_t *dst = which ? VbT : KbT;
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[(q8 + e) * 64 + s] = f2bf(sc * bf16f(e8[e]));
            }
            // sweep operands formed elementwise: QE, KT (2 x 4 lane slots each) and P (2 x 2)
            for (int slot = tid; slot < 2 * 4 * 64 * 2 + 2 * 2 * 64; slot += 256) {
                float vals[16];
                const int sl = slot & 63, sh = sl >> 5, s32 = sl & 31;
                if (slot < 2 * 4 * 64) {                       // QE[mb][w][lane]
                    const int mb = slot >> 8, w = (slot >> 6) & 3;
                    const int t = 32 * mb + s32;
                    const float e = __expf(gj[t]);
#pragma unroll
                    for (int i = 0; i < 16; ++i) vals[i] = e * bf16f(qkr[t * 2 * DKP + 32 * w + kx(i, sh)]);
                    store16(blk + kOffQE + (size_t)slot * 16, vals);
                } else if (slot < 2 * 2 * 4 * 64) {           // KT[mb][w][lane]
                    const int s2 = slot - 2 * 4 * 64;
                    const int mb = s2 >> 8, w = (s2 >> 6) & 3;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int t = 32 * mb + kx(i, sh);
                        vals[i] = __expf(gL - gj[t]) * bf16f(qkr[t * 2 * DKP + DKP + 32 * w + s32]);
                    }
                    store16(blk + kOffKT + (size_t)s2 * 16, vals);
                } else {                                       // P[mb][mbk][lane]
                    const int s3 = slot - 2 * 2 * 4 * 64;
                    const int mb = s3 >> 7, mbk = (s3 >> 6) & 1;
                    const int t = 32 * mb + s32;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int s = 32 * mbk + kx(i, sh);
                        vals[i] = (s <= t && t < L) ? __expf(gj[t] - gj[s]) * Sqk[t * 64 + s] : 0.0f;
                    }
                    store16(blk + kOffP + (size_t)s3 * 16, vals);
                }
            }
            if (tid == 0) X.el[(size_t)(cid0 + c) * hv + h] = __expf(gL);
            lds_barrier();
            // W^T = Kb^T T^T and U~ = T Vb: wave w does 4 of the 16 output blocks
            {
                const uint16_t *Tj = Tb + jj * 64 * 64;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int b = wave * 4 + q;              // 0..7: W^T (kb, bi); 8..15: U~ (bi, tile)
                    const bool isw = b < 8;
                    const int x = (b & 7) >> 1, y = b & 1;   // W^T: kb = x, bi = y; U~: tile = x, bi = y
                    f16v acc = {};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int ko = 16 * ks + 8 * hh;
                        const bf8v a = isw ? lds8(KbT + (32 * x + l32) * 64 + ko) : lds8(Tj + (32 * y + l32) * 64 + ko);
                        const bf8v bb = isw ? lds8(Tj + (32 * y + l32) * 64 + ko) : lds8(VbT + (32 * x + l32) * 64 + ko);
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
                    }
                    float vals[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) vals[i] = acc[i];
                    // W^T block (kb, bi): lane l holds W[32 bi + l32][32 kb + kx(i)] = W[mb=bi][w=kb]
                    // U~ block (bi, tile): lane l holds U~[32 bi + kx(i)][32 tile + l32] = UT[mb=bi][tile]
                    const size_t off = isw ? kOffW + ((size_t)(y * 4 + x) * 64 + lane) * 16
                                           : kOffUT + ((size_t)(y * 4 + x) * 64 + lane) * 16;
                    store16(blk + off, vals);
                }
            }
            lds_barrier();
        }
    }
}

// ---------------------------------------------------------------- sweep
__device__ __forceinline__ float bfat(const uint4 (&v)[2], int i)
{
    const uint4 &u = v[i >> 3];
    const int k = (i & 7) >> 1;
    const uint32_t w = k == 0 ? u.x : k == 1 ? u.y : k == 2 ? u.z : u.w;
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
}

__device__ __forceinline__ void ld2(uint4 (&v)[2], const uint16_t *p)
{
    v[0] = reinterpret_cast<const uint4 *>(p)[0];
    v[1] = reinterpret_cast<const uint4 *>(p)[1];
}

__device__ __forceinline__ f16v mfma_f32(float a, float b, f16v c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__global__ void __launch_bounds__(256) sweep_kernel(const Ctx X)
{
    extern __shared__ float smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int hv = X.P.hv, n = X.P.n_seqs;
    const int ntile = DKP / TILE;
    const int tile = blockIdx.x % ntile;
    const int h = (blockIdx.x / ntile) % hv;
    const int slot = blockIdx.x / (ntile * hv);

    float *red_u = smem;                     // [4 waves][2][16][64]
    float *red_o = red_u + 4 * 2 * 16 * 64;  // [4 waves][2][16][64]
    int *order = reinterpret_cast<int *>(red_o + 4 * 2 * 16 * 64);   // [256] prompt of each rank

    // prompts by decreasing length (ties by index), so the longest chains start first
    int pidx = slot;
    if (n <= 256) {
        if (tid < n) {
            const int len = X.P.seq_start[tid + 1] - X.P.seq_start[tid];
            int rank = 0;
            for (int q = 0; q < n; ++q) {
                const int lq = X.P.seq_start[q + 1] - X.P.seq_start[q];
                rank += (lq > len) || (lq == len && q < tid);
            }
            order[rank] = tid;
        }
        lds_barrier();
        pidx = order[slot];
    }
    int s0, s1, cid0;
    if (!prompt_chunks(X, pidx, s0, s1, cid0)) return;
    const int len = s1 - s0;
    const int col = tile * TILE + l32;

    // this wave's 32 state rows x 32 columns, in accumulator layout:
    // register i of lane l is M[32 w + kx(i)][col]
    float *st = X.P.state + ((size_t)pidx * hv + h) * DKP * DKP;
    f16v M;
#pragma unroll
    for (int i = 0; i < 16; ++i) M[i] = st[(size_t)(32 * wave + kx(i, hh)) * DKP + col];

    const int nck = (len + kChunk - 1) / kChunk;
    const size_t cstride = (size_t)hv * kBlockElems;
    const uint16_t *blk = X.blk + ((size_t)cid0 * hv + h) * kBlockElems;
    const int mbk = wave >> 1, i0 = 8 * (wave & 1);
    // this lane's operands of the current chunk
    uint4 Wo[2][2], QEo[2][2], KTo[2][2], UTo[2][2], Po[2];
    if (nck > 0) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            ld2(Wo[mb], blk + kOffW + ((size_t)(mb * 4 + wave) * 64 + lane) * 16);
            ld2(UTo[mb], blk + kOffUT + ((size_t)(mb * 4 + tile) * 64 + lane) * 16);
            ld2(QEo[mb], blk + kOffQE + ((size_t)(mb * 4 + wave) * 64 + lane) * 16);
            Po[mb] = *reinterpret_cast<const uint4 *>(blk + kOffP + ((size_t)(mb * 2 + mbk) * 64 + lane) * 16 + i0);
            ld2(KTo[mb], blk + kOffKT + ((size_t)(mb * 4 + wave) * 64 + lane) * 16);
        }
    }
    for (int c = 0; c < nck; ++c) {
        const int r0 = s0 + c * kChunk;
        const int L = min(kChunk, s1 - r0);
        const bool more = c + 1 < nck;
        const uint16_t *bn = blk + (size_t)(c + 1) * cstride;
        const float eL = X.el[(size_t)(cid0 + c) * hv + h];

        // partial of W M0 over this wave's 32 state rows
        f16v up[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            up[mb] = f16v{};
#pragma unroll
            for (int i = 0; i < 16; ++i) up[mb] = mfma_f32(bfat(Wo[mb], i), M[i], up[mb]);
            if (more) ld2(Wo[mb], bn + kOffW + ((size_t)(mb * 4 + wave) * 64 + lane) * 16);
#pragma unroll
            for (int i = 0; i < 16; ++i) red_u[((wave * 2 + mb) * 16 + i) * 64 + lane] = up[mb][i];
        }
        lds_barrier();

        // U = U~ - W M0 (every wave keeps all of it, in accumulator layout)
        f16v U[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = red_u[((0 * 2 + mb) * 16 + i) * 64 + lane];
                s += red_u[((1 * 2 + mb) * 16 + i) * 64 + lane];
                s += red_u[((2 * 2 + mb) * 16 + i) * 64 + lane];
                s += red_u[((3 * 2 + mb) * 16 + i) * 64 + lane];
                U[mb][i] = bfat(UTo[mb], i) - s;
            }
            if (more) ld2(UTo[mb], bn + kOffUT + ((size_t)(mb * 4 + tile) * 64 + lane) * 16);
        }

        // partial of O: (e^gamma q) M0 over this wave's state rows, plus a quarter of P U
        f16v op[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            op[mb] = f16v{};
#pragma unroll
            for (int i = 0; i < 16; ++i) op[mb] = mfma_f32(bfat(QEo[mb], i), M[i], op[mb]);
            const uint4 pv[2] = {Po[mb], Po[mb]};
#pragma unroll
            for (int i = 0; i < 8; ++i) op[mb] = mfma_f32(bfat(pv, i), U[mbk][i0 + i], op[mb]);
            if (more) {
                ld2(QEo[mb], bn + kOffQE + ((size_t)(mb * 4 + wave) * 64 + lane) * 16);
                Po[mb] = *reinterpret_cast<const uint4 *>(bn + kOffP + ((size_t)(mb * 2 + mbk) * 64 + lane) * 16 + i0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) red_o[((wave * 2 + mb) * 16 + i) * 64 + lane] = op[mb][i];
        }
        lds_barrier();

        // O rows: wave w sums the four partials of registers [i0, i0 + 8) of block mbk
#pragma unroll
        for (int i = i0; i < i0 + 8; ++i) {
            const int row = 32 * mbk + kx(i, hh);
            float s = red_o[((0 * 2 + mbk) * 16 + i) * 64 + lane];
            s += red_o[((1 * 2 + mbk) * 16 + i) * 64 + lane];
            s += red_o[((2 * 2 + mbk) * 16 + i) * 64 + lane];
            s += red_o[((3 * 2 + mbk) * 16 + i) * 64 + lane];
            if (row < L) X.P.out[((size_t)(r0 + row) * hv + h) * DKP + col] = s;
        }

        // M <- e^{gamma_L} M0 + (e^{gamma_L - gamma} k)^T U on this wave's rows
#pragma unroll
        for (int i = 0; i < 16; ++i) M[i] *= eL;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) M = mfma_f32(bfat(KTo[mb], i), U[mb][i], M);
            if (more) ld2(KTo[mb], bn + kOffKT + ((size_t)(mb * 4 + wave) * 64 + lane) * 16);
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) st[(size_t)(32 * wave + kx(i, hh)) * DKP + col] = M[i];

    // the prompt's conv tail: its last three raw rows, continuing into the old
    // tail when the prompt is shorter (one workgroup a prompt, read then write)
    if (h == 0 && tile == 0 && len > 0) {
        const int C = X.P.C;
        uint16_t *tl = X.P.conv_tail + (size_t)pidx * 3 * C;
        for (int ch = tid; ch < C; ch += 256) {
            uint16_t nt[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int m = len - 3 + j;   // local row of new tail row j
                nt[j] = m >= 0 ? X.P.qkv[(size_t)(s0 + m) * C + ch] : tl[(size_t)(m + 3) * C + ch];
            }
#pragma unroll
            for (int j = 0; j < 3; ++j) tl[(size_t)j * C + ch] = nt[j];
        }
    }
}

size_t prologue_lds(int r)
{
    const size_t nch = (size_t)(2 + r) * DKP;
    return sizeof(float) * PRO_ROWS * 2 * DKP + sizeof(float) * 4 * nch +
           sizeof(uint16_t) * (PRO_ROWS + 3) * nch + sizeof(int) * 2 * PRO_ROWS;
}
size_t intra_lds()
{
    return sizeof(uint16_t) * 64 * 2 * DKP + sizeof(float) * (2 * 64 * 64 + HB * 64 * 64 + 2 * HB * 64) +
           sizeof(uint16_t) * HB * 64 * 64;
}
size_t sweep_lds() { return sizeof(float) * (2 * 4 * 2 * 16 * 64) + sizeof(int) * 256; }

template <typename K>
hipError_t allow(K kernel, size_t bytes)
{
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

PrefillLayout prefill_layout(int hk, int hv, int dk, int dv, int n_seqs, int T)
{
    PrefillLayout Lo = {};
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
    const size_t t = (size_t)T;
    // each prompt adds at most one partial chunk to floor(T / 64) whole ones
    Lo.max_chunks_total = T / kChunk + n_seqs;
    const size_t nc = (size_t)Lo.max_chunks_total;
    Lo.qk = take(t * hk * 2 * dk * 2);
    Lo.v = take(t * hv * dv * 2);
    Lo.g = take(t * hv * 4);
    Lo.be = take(t * hv * 4);
    Lo.blk = take(nc * hv * kBlockElems * 2);
    Lo.el = take(nc * hv * 4);
    Lo.total = o;
    return Lo;
}

bool prefill_supported(int hk, int hv, int dk, int dv)
{
    return dk == DKP && dv == DKP && hk > 0 && hv % hk == 0 && hv / hk <= 8;
}

size_t prefill_workspace_bytes(int hk, int hv, int dk, int dv, int n_seqs, int total_rows)
{
    if (!prefill_supported(hk, hv, dk, dv)) return 0;
    return prefill_layout(hk, hv, dk, dv, n_seqs, total_rows).total;
}

hipError_t launch_prefill(const PrefillArgs &P, hipStream_t stream)
{
    const PrefillLayout Lo = prefill_layout(P.hk, P.hv, P.dk, P.dv, P.n_seqs, P.total_rows);
    char *ws = static_cast<char *>(P.workspace);
    Ctx X;
    X.P = P;
    X.r = P.hv / P.hk;
    X.max_chunks = (P.max_len + kChunk - 1) / kChunk;
    X.nc_total = Lo.max_chunks_total;
    X.qk = reinterpret_cast<uint16_t *>(ws + Lo.qk);
    X.v = reinterpret_cast<uint16_t *>(ws + Lo.v);
    X.g = reinterpret_cast<float *>(ws + Lo.g);
    X.be = reinterpret_cast<float *>(ws + Lo.be);
    X.blk = reinterpret_cast<uint16_t *>(ws + Lo.blk);
    X.el = reinterpret_cast<float *>(ws + Lo.el);

    static const hipError_t e1 = allow(prologue_kernel, prologue_lds(8));
    static const hipError_t e2 = allow(intra_kernel, intra_lds());
    static const hipError_t e3 = allow(sweep_kernel, sweep_lds());
    if (e1 != hipSuccess) return e1;
    if (e2 != hipSuccess) return e2;
    if (e3 != hipSuccess) return e3;

    hipLaunchKernelGGL(prologue_kernel, dim3((P.total_rows + PRO_ROWS - 1) / PRO_ROWS, P.hk), dim3(256),
                       prologue_lds(X.r), stream, X);
    hipLaunchKernelGGL(intra_kernel, dim3((unsigned)P.n_seqs * X.max_chunks, P.hk), dim3(256), intra_lds(), stream, X);
    hipLaunchKernelGGL(sweep_kernel, dim3((unsigned)P.n_seqs * P.hv * (DKP / TILE)), dim3(256), sweep_lds(), stream, X);
    return hipGetLastError();
}

}  // namespace gdn
