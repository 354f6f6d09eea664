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
//             (v_mfma_f32_32x32x16_bf16), then per value head gamma, the
//             fp32 triangular solve for T (one wave, one column a lane), P,
//             and W, U~ on bf16 MFMA.  Independent across chunks.
//   sweep     per (prompt, value head, 32 state columns), 4 waves, each
//             holding 32 rows of the state as an fp32 MFMA accumulator: the
//             state contractions U~ - W M0, (e^gamma q) M0, P U and the
//             update (e^{gamma_L - gamma} k)^T U run on fp32 MFMA
//             (v_mfma_f32_32x32x2_f32) with the accumulator itself as the
//             B operand; partial sums over the four row blocks meet in LDS.
//             Sequential over the prompt's chunks; the state never leaves
//             the chip between them.
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

struct Ctx {
    PrefillArgs P;
    int r;                      // value heads per key head
    int max_chunks;             // chunks of the longest prompt
    uint16_t *qk, *v, *w, *u, *p;
    float *g, *be, *gam;
};

__device__ __forceinline__ bool prompt_ok(const Ctx &X, int p, int &s0, int &s1)
{
    s0 = X.P.seq_start[p];
    s1 = X.P.seq_start[p + 1];
    return s0 >= 0 && s1 >= s0 && s1 <= X.P.total_rows && s1 - s0 <= X.P.max_len;
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
    uint16_t *raw = reinterpret_cast<uint16_t *>(act + PRO_ROWS * 2 * DKP);  // [PRO_ROWS + 3][nch]
    int *rstart = reinterpret_cast<int *>(raw + (PRO_ROWS + 3) * nch);     // [PRO_ROWS]
    int *rprompt = rstart + PRO_ROWS;                                      // [PRO_ROWS]

    // prompt of each row: the last p with seq_start[p] <= t, if t < seq_start[p + 1]
    if (tid < nrows) {
        const int t = t0 + tid;
        int lo = 0, hi = X.P.n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (X.P.seq_start[mid] <= t) lo = mid; else hi = mid - 1;
        }
        int s0, s1;
        const bool ok = prompt_ok(X, lo, s0, s1) && s0 <= t && t < s1;
        rstart[tid] = ok ? s0 : -1;
        rprompt[tid] = lo;
    }
    // stage raw rows t0-3 .. t0+nrows-1 of this key head's channels
    const int cpr = nch / 8;
    for (int idx = tid; idx < (nrows + 3) * cpr; idx += 256) {
        const int j = idx / cpr;
        const int lc = (idx - j * cpr) * 8;
        const int u = t0 - 3 + j;
        if (u >= 0)
            *reinterpret_cast<uint4 *>(raw + j * nch + lc) =
                *reinterpret_cast<const uint4 *>(X.P.qkv + (size_t)u * C + pro_channel(X, kh, lc));
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
    // conv + SiLU: q/k into LDS for the norms, v straight out as bf16
    for (int idx = tid; idx < nrows * nch; idx += 256) {
        const int i = idx / nch;
        const int ch = idx - i * nch;
        const int rs = rstart[i];
        if (rs < 0) continue;
        const int t = t0 + i;
        const int gc = pro_channel(X, kh, ch);
        const float4 w = *reinterpret_cast<const float4 *>(X.P.conv_w + (size_t)gc * 4);
        float x[4];
#pragma unroll
        for (int d = 3; d >= 0; --d) {
            const int src = t - d;
            const uint16_t bits = src >= rs ? raw[(i + 3 - d) * nch + ch]
                                            : X.P.conv_tail[((size_t)rprompt[i] * 3 + (3 + src - rs)) * C + gc];
            x[3 - d] = bf16f(bits);
        }
        float y = w.x * x[0];
        y = fmaf(w.y, x[1], y);
        y = fmaf(w.z, x[2], y);
        y = fmaf(w.w, x[3], y);
        const float a = silu_f(y);
        if (ch < 2 * DKP)
            act[i * 2 * DKP + ch] = a;
        else
            X.v[(size_t)t * X.P.hv * DKP + (size_t)kh * X.r * DKP + (ch - 2 * DKP)] = f2bf(a);
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
// 8 consecutive bf16 of a workspace row as an MFMA operand (zeros past the chunk).
__device__ __forceinline__ bf8v load8(const uint16_t *p, bool ok)
{
    uint4 raw = ok ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
    return __builtin_bit_cast(bf8v, raw);
}

__device__ __forceinline__ bf8v lds8(const uint16_t *p) { return __builtin_bit_cast(bf8v, *reinterpret_cast<const uint4 *>(p)); }

constexpr int HB = 3;   // value heads whose triangular solves run side by side

__global__ void __launch_bounds__(256) intra_kernel(const Ctx X)
{
    extern __shared__ float smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int kh = blockIdx.y;
    const int pidx = blockIdx.x / X.max_chunks, c = blockIdx.x - pidx * X.max_chunks;
    int s0, s1;
    if (!prompt_ok(X, pidx, s0, s1)) return;
    const int r0 = s0 + c * kChunk;
    if (r0 >= s1) return;
    const int L = min(kChunk, s1 - r0);
    const int hv = X.P.hv, hk = X.P.hk;

    float *Skk = smem;                          // [64][64]
    float *Sqk = Skk + 64 * 64;                 // [64][64]
    float *An = Sqk + 64 * 64;                  // [HB][64][64] -A, later KbT / VbT
    uint16_t *Tb = reinterpret_cast<uint16_t *>(An + HB * 64 * 64);   // [HB][64][64] bf16
    float *gam = reinterpret_cast<float *>(Tb + HB * 64 * 64);       // [HB][64]
    float *bet = gam + HB * 64;                                        // [HB][64]
    uint16_t *KbT = reinterpret_cast<uint16_t *>(An);                  // [128][64]
    uint16_t *VbT = KbT + 128 * 64;                                    // [128][64]

    // K K^T and Q K^T: wave w computes the 32 x 32 block (w >> 1, w & 1) of both
    {
        const int bi = wave >> 1, bj = wave & 1;
        const int ra = 32 * bi + l32, rb = 32 * bj + l32;
        const uint16_t *qa = X.qk + ((size_t)(r0 + ra) * hk + kh) * 2 * DKP;
        const uint16_t *kb = X.qk + ((size_t)(r0 + rb) * hk + kh) * 2 * DKP + DKP;
        f16v kk = {}, qk = {};
#pragma unroll
        for (int ks = 0; ks < DKP / 16; ++ks) {
            const int ko = 16 * ks + 8 * hh;
            const bf8v ak = load8(qa + DKP + ko, ra < L);
            const bf8v aq = load8(qa + ko, ra < L);
            const bf8v bk = load8(kb + ko, rb < L);
            kk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, bk, kk, 0, 0, 0);
            qk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, qk, 0, 0, 0);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 32 * bi + 8 * (rr >> 2) + 4 * hh + (rr & 3);
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
            if (lane < L) X.gam[o] = gl;
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
#pragma unroll
            for (int t = 0; t < 64; ++t) {
                float acc = (t == lane) ? 1.0f : 0.0f;
#pragma unroll
                for (int s4 = 0; s4 < 64; s4 += 4) {
                    if (s4 < t) {
                        const float4 a4 = *reinterpret_cast<const float4 *>(Aj + t * 64 + s4);
                        acc = fmaf(a4.x, Tc[s4], acc);
                        if (s4 + 1 < t) acc = fmaf(a4.y, Tc[s4 + 1], acc);
                        if (s4 + 2 < t) acc = fmaf(a4.z, Tc[s4 + 2], acc);
                        if (s4 + 3 < t) acc = fmaf(a4.w, Tc[s4 + 3], acc);
                    }
                }
                Tc[t] = acc;
            }
            uint16_t *Tj = Tb + wave * 64 * 64;
#pragma unroll
            for (int t = 0; t < 64; ++t) Tj[t * 64 + lane] = f2bf(Tc[t]);
        } else if (wave == 3) {
            // P_ts = e^{gamma_t - gamma_s} (q_t . k_s) for s <= t, row `lane`
            const int t = lane;
            if (t < L) {
                for (int jj = 0; jj < nh; ++jj) {
                    const int h = kh * X.r + j0 + jj;
                    const float *gj = gam + jj * 64;
                    const float gt = gj[t];
                    uint16_t *dst = X.p + ((size_t)(r0 + t) * hv + h) * 64;
                    for (int s8 = 0; s8 < 64; s8 += 8) {
                        uint16_t pk[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int s = s8 + e;
                            pk[e] = s <= t ? f2bf(__expf(gt - gj[s]) * Sqk[t * 64 + s]) : (uint16_t)0;
                        }
                        *reinterpret_cast<uint4 *>(dst + s8) = *reinterpret_cast<const uint4 *>(pk);
                    }
                }
            }
        }
        lds_barrier();

        for (int jj = 0; jj < nh; ++jj) {
            const int h = kh * X.r + j0 + jj;
            const float *gj = gam + jj * 64, *bj = bet + jj * 64;
            // KbT[k][s] = beta_s e^{gamma_s} k_s[k],  VbT[c][s] = beta_s v_s[c]
            for (int idx = tid; idx < 64 * 16 * 2; idx += 256) {
                const int which = idx >= 64 * 16;
                const int id = idx - which * 64 * 16;
                const int s = id >> 4, q8 = (id & 15) * 8;
                uint4 raw = make_uint4(0, 0, 0, 0);
                if (s < L)
                    raw = *reinterpret_cast<const uint4 *>(
                        which ? X.v + ((size_t)(r0 + s) * hv + h) * DKP + q8
                              : X.qk + ((size_t)(r0 + s) * hk + kh) * 2 * DKP + DKP + q8);
                const uint16_t *e8 = reinterpret_cast<const uint16_t *>(&raw);
                const float sc = which ? bj[s] : bj[s] * __expf(gj[s]);
                uint16_t *dst = which ? VbT : KbT;
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[(q8 + e) * 64 + s] = f2bf(sc * bf16f(e8[e]));
            }
            lds_barrier();
            // W = T Kb and U~ = T Vb: wave w does one 32-row half of one of them
            {
                const int which = wave >> 1, bi = wave & 1;
                const uint16_t *Tj = Tb + jj * 64 * 64;
                const uint16_t *BT = which ? VbT : KbT;
                uint16_t *dst = which ? X.u : X.w;
#pragma unroll
                for (int bjc = 0; bjc < 4; ++bjc) {
                    f16v acc = {};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int ko = 16 * ks + 8 * hh;
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(Tj + (32 * bi + l32) * 64 + ko),
                                                                      lds8(BT + (32 * bjc + l32) * 64 + ko), acc,
                                                                      0, 0, 0);
                    }
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        const int row = 32 * bi + 8 * (rr >> 2) + 4 * hh + (rr & 3);
                        if (row < L) dst[((size_t)(r0 + row) * hv + h) * DKP + 32 * bjc + l32] = f2bf(acc[rr]);
                    }
                }
            }
            lds_barrier();
        }
    }
}

// ---------------------------------------------------------------- sweep
// 4 consecutive bf16 of a workspace row as fp32 (zeros past the chunk).
__device__ __forceinline__ float4 load4(const uint16_t *p, bool ok)
{
    if (!ok) return make_float4(0.f, 0.f, 0.f, 0.f);
    const uint2 r = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
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
    const int hv = X.P.hv, hk = X.P.hk;
    const int ntile = DKP / TILE;
    const int tile = blockIdx.x % ntile;
    const int h = (blockIdx.x / ntile) % hv;
    const int pidx = blockIdx.x / (ntile * hv);
    int s0, s1;
    if (!prompt_ok(X, pidx, s0, s1)) return;
    const int len = s1 - s0;
    const int kh = h / X.r;
    const int col = tile * TILE + l32;

    float *red_u = smem;                     // [4 waves][2][16][64]
    float *red_o = red_u + 4 * 2 * 16 * 64;  // [4 waves][2][16][64]
    float *gbuf = red_o + 4 * 2 * 16 * 64;   // [2][64]

    // this wave's 32 state rows x 32 columns, in accumulator layout:
    // register i of lane l is M[32 w + 8 (i / 4) + 4 (l / 32) + i % 4][col]
    float *st = X.P.state + ((size_t)pidx * hv + h) * DKP * DKP;
    f16v M;
#pragma unroll
    for (int i = 0; i < 16; ++i) M[i] = st[(size_t)(32 * wave + 8 * (i >> 2) + 4 * hh + (i & 3)) * DKP + col];

    const int nck = (len + kChunk - 1) / kChunk;
    for (int c = 0; c < nck; ++c) {
        const int r0 = s0 + c * kChunk;
        const int L = min(kChunk, s1 - r0);
        float *gb = gbuf + (c & 1) * 64;
        if (wave == 0) gb[lane] = X.gam[(size_t)(r0 + min(lane, L - 1)) * hv + h];

        // partial of W M0 over this wave's 32 state rows (chunk rows 32 mb + l % 32)
        f16v up[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int row = 32 * mb + l32;
            const uint16_t *wr = X.w + ((size_t)(r0 + row) * hv + h) * DKP + 32 * wave + 4 * hh;
            up[mb] = f16v{};
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 a4 = load4(wr + 8 * g4, row < L);
                up[mb] = mfma_f32(a4.x, M[4 * g4 + 0], up[mb]);
                up[mb] = mfma_f32(a4.y, M[4 * g4 + 1], up[mb]);
                up[mb] = mfma_f32(a4.z, M[4 * g4 + 2], up[mb]);
                up[mb] = mfma_f32(a4.w, M[4 * g4 + 3], up[mb]);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) red_u[((wave * 2 + mb) * 16 + i) * 64 + lane] = up[mb][i];
        }
        lds_barrier();

        // U = U~ - W M0 (every wave keeps all of it, in accumulator layout)
        f16v U[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
                float s = red_u[((0 * 2 + mb) * 16 + i) * 64 + lane];
                s += red_u[((1 * 2 + mb) * 16 + i) * 64 + lane];
                s += red_u[((2 * 2 + mb) * 16 + i) * 64 + lane];
                s += red_u[((3 * 2 + mb) * 16 + i) * 64 + lane];
                const float ut = row < L ? bf16f(X.u[((size_t)(r0 + row) * hv + h) * DKP + col]) : 0.0f;
                U[mb][i] = ut - s;
            }

        // partial of O: (e^gamma q) M0 over this wave's state rows, plus a quarter of P U
        f16v op[2];
        const int mbk = wave >> 1, i0 = 8 * (wave & 1);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int row = 32 * mb + l32;
            const bool ok = row < L;
            const float eg = __expf(gb[row]);
            const uint16_t *qr = X.qk + ((size_t)(r0 + row) * hk + kh) * 2 * DKP + 32 * wave + 4 * hh;
            op[mb] = f16v{};
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 a4 = load4(qr + 8 * g4, ok);
                op[mb] = mfma_f32(eg * a4.x, M[4 * g4 + 0], op[mb]);
                op[mb] = mfma_f32(eg * a4.y, M[4 * g4 + 1], op[mb]);
                op[mb] = mfma_f32(eg * a4.z, M[4 * g4 + 2], op[mb]);
                op[mb] = mfma_f32(eg * a4.w, M[4 * g4 + 3], op[mb]);
            }
            const uint16_t *pr = X.p + ((size_t)(r0 + row) * hv + h) * 64 + 32 * mbk + 4 * hh;
#pragma unroll
            for (int g4 = 0; g4 < 2; ++g4) {
                const int i = i0 + 4 * g4;
                const float4 a4 = load4(pr + 8 * (i >> 2), ok);
                op[mb] = mfma_f32(a4.x, U[mbk][i + 0], op[mb]);
                op[mb] = mfma_f32(a4.y, U[mbk][i + 1], op[mb]);
                op[mb] = mfma_f32(a4.z, U[mbk][i + 2], op[mb]);
                op[mb] = mfma_f32(a4.w, U[mbk][i + 3], op[mb]);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) red_o[((wave * 2 + mb) * 16 + i) * 64 + lane] = op[mb][i];
        }
        lds_barrier();

        // O rows: wave w sums the four partials of registers [i0, i0 + 8) of block mbk
#pragma unroll
        for (int i = i0; i < i0 + 8; ++i) {
            const int row = 32 * mbk + 8 * (i >> 2) + 4 * hh + (i & 3);
            float s = red_o[((0 * 2 + mbk) * 16 + i) * 64 + lane];
            s += red_o[((1 * 2 + mbk) * 16 + i) * 64 + lane];
            s += red_o[((2 * 2 + mbk) * 16 + i) * 64 + lane];
            s += red_o[((3 * 2 + mbk) * 16 + i) * 64 + lane];
            if (row < L) X.P.out[((size_t)(r0 + row) * hv + h) * DKP + col] = s;
        }

        // M <- e^{gamma_L} M0 + (e^{gamma_L - gamma} k)^T U on this wave's rows
        const float gL = gb[L - 1];
        const float eL = __expf(gL);
#pragma unroll
        for (int i = 0; i < 16; ++i) M[i] *= eL;
        const uint16_t *kc = X.qk + (size_t)kh * 2 * DKP + DKP + 32 * wave + l32;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
                const float a = row < L ? __expf(gL - gb[row]) * bf16f(kc[(size_t)(r0 + row) * hk * 2 * DKP]) : 0.0f;
                M = mfma_f32(a, U[mb][i], M);
            }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) st[(size_t)(32 * wave + 8 * (i >> 2) + 4 * hh + (i & 3)) * DKP + col] = M[i];

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

size_t prologue_lds(int r) { return sizeof(float) * PRO_ROWS * 2 * DKP + sizeof(uint16_t) * (PRO_ROWS + 3) * (2 + r) * DKP + sizeof(int) * 2 * PRO_ROWS; }
size_t intra_lds() { return sizeof(float) * (2 * 64 * 64 + HB * 64 * 64 + 2 * HB * 64) + sizeof(uint16_t) * HB * 64 * 64; }
size_t sweep_lds() { return sizeof(float) * (2 * 4 * 2 * 16 * 64 + 2 * 64); }

template <typename K>
hipError_t allow(K kernel, size_t bytes)
{
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

PrefillLayout prefill_layout(int hk, int hv, int dk, int dv, int T)
{
    PrefillLayout Lo = {};
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
    const size_t t = (size_t)T;
    Lo.qk = take(t * hk * 2 * dk * 2);
    Lo.v = take(t * hv * dv * 2);
    Lo.g = take(t * hv * 4);
    Lo.be = take(t * hv * 4);
    Lo.gam = take(t * hv * 4);
    Lo.w = take(t * hv * dk * 2);
    Lo.u = take(t * hv * dv * 2);
    Lo.p = take(t * hv * kChunk * 2);
    Lo.total = o;
    return Lo;
}

bool prefill_supported(int hk, int hv, int dk, int dv)
{
    return dk == DKP && dv == DKP && hk > 0 && hv % hk == 0 && hv / hk <= 8;
}

size_t prefill_workspace_bytes(int hk, int hv, int dk, int dv, int, int total_rows)
{
    if (!prefill_supported(hk, hv, dk, dv)) return 0;
    return prefill_layout(hk, hv, dk, dv, total_rows).total;
}

hipError_t launch_prefill(const PrefillArgs &P, hipStream_t stream)
{
    const PrefillLayout Lo = prefill_layout(P.hk, P.hv, P.dk, P.dv, P.total_rows);
    char *ws = static_cast<char *>(P.workspace);
    Ctx X;
    X.P = P;
    X.r = P.hv / P.hk;
    X.max_chunks = (P.max_len + kChunk - 1) / kChunk;
    X.qk = reinterpret_cast<uint16_t *>(ws + Lo.qk);
    X.v = reinterpret_cast<uint16_t *>(ws + Lo.v);
    X.g = reinterpret_cast<float *>(ws + Lo.g);
    X.be = reinterpret_cast<float *>(ws + Lo.be);
    X.gam = reinterpret_cast<float *>(ws + Lo.gam);
    X.w = reinterpret_cast<uint16_t *>(ws + Lo.w);
    X.u = reinterpret_cast<uint16_t *>(ws + Lo.u);
    X.p = reinterpret_cast<uint16_t *>(ws + Lo.p);

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
