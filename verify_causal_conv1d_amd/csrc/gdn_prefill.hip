// Chunked prompt pass of libgdn (gfx950): the gated delta rule in chunkwise
// WY form, chunks of 64 rows that never cross prompts.
//
// Within a chunk that starts from state M0 (M = S^T, [dk][dv]), with
// g_t = log alpha_t and gamma_t = g_1 + ... + g_t (in-chunk),
//   A_tj = beta_t e^{gamma_t - gamma_j} k_t.k_j (j < t),  T = (I + A)^-1,
//   W = T (beta e^gamma k),  U~ = T (beta v),  U = U~ - W M0,
//   P_tj = e^{gamma_t - gamma_j} q_t.k_j (j <= t),
//   O = (e^gamma q) M0 + P U,
//   M_next = e^{gamma_L} M0 + (e^{gamma_L - gamma} k)^T U.
// (The derivation unrolls M_t = alpha_t M_{t-1} + k_t d_t^T with
// d_t = beta_t (v_t - alpha_t M_{t-1}^T k_t) over the chunk; the gated delta
// rule is Yang, Kautz and Hatamizadeh, "Gated Delta Networks", 2024.)
// The parallel per-chunk kernels form every operand that does not involve
// the state; the sequential sweep forms [W; e^gamma q] M0 and the update with
// the fp32 operand (M0, U) split exactly into three bf16 terms (products as
// exact as on fp32 MFMA, at the bf16 matrix rate), and P U (an in-chunk
// product of the chunk's own deltas U, which only the sweep knows) on bf16
// MFMA, and writes each output row once.
//
// Three launches on the caller's stream:
//   qk        per (chunk, key head), independent: the causal conv (taps from
//             the prompt's own earlier rows or its tail) + SiLU of the chunk's
//             q and k channels straight from the packed rows, the q/k L2 norms
//             over the 16 lanes of a head, K K^T and Q K^T on bf16 MFMA, and
//             the transposed k^ fragments: what the r value heads of a key
//             head share, formed once and left in the lane order the next
//             kernel's waves read.
//   intra     per (chunk, value head), independent: the gates, T by 16 x 16
//             blocks (fp32 forward substitution on the diagonal, fp32 MFMA
//             off it), the conv + SiLU of the chunk's v channels, then W^T and
//             U~ on bf16 MFMA, and P as it is.  v is transposed by an exact
//             MFMA with a 0/1 selection operand (k^ comes transposed from
//             qk), and every product takes a k order in which one product's
//             accumulator registers are the next one's operand, so nothing is
//             transposed through LDS; products are formed transposed where
//             that puts each lane's values where the sweep's lanes read them,
//             and everything leaves in that order.
//   sweep     per (prompt, value head, 32 state columns: two 16-column
//             tiles), 4 waves; wave w keeps state rows [32w, 32w + 32) of
//             both tiles as four fp32 16 x 16 MFMA accumulators and leaves
//             their three bf16 terms in LDS, where every wave reads all of
//             M0.  Per chunk and tile: rows [16w, 16w + 16) of W M0 and
//             (e^gamma q) M0 over the 128 state rows, U = U~ - W M0 shared
//             through LDS (rounded for P U, in terms for the update),
//             O = (e^gamma q) M0 + P U, then M = e^{gamma_L} M + K~^T U on the
//             wave's rows, all on v_mfma_f32_16x16x32_bf16; the chunk's
//             operands serve both tiles.  Sequential over the prompt's
//             chunks, operands of chunk c + 1 fetched while chunk c
//             computes; the state never leaves the chip.  The 4 tile pairs
//             of the r value heads of one (prompt, key head) share operands
//             and are placed on one XCD (workgroup i runs on XCD i mod 8) so
//             that they meet in that XCD's L2; prompts run longest first.
// The prompt's final state replaces the stream's state, and its last three raw
// rows (or a mix with the old tail for prompts shorter than three rows) its
// conv tail, in place, both by the sweep, after every read of the old tail (prompt passes update the stream in place: page
// "perf(qwen3_5 cuda): deliver the first token before drafting", commit note
// on tree-shaped verify windows).
#include "gdn_device.h"
#include "gdn_prefill.h"

namespace gdn {
namespace {

constexpr int D = 128;          // dk = dv of this pass
constexpr int NTILE = D / 16;   // 16-column state tiles of a head

// A chunk-head block of sweep operands (bf16), every sub-array in lane order
// [..][64 lanes][values]; lane l = (l16, g4) = (l & 15, l >> 4), and
// accumulator register i of a 16x16 block holds row 4 g4 + i, column l16.
//   W  [w 4][s 4][l][8]         W[16w + l16][16kb + 4g4 + (e & 3)] with
//        kb = 2s + (e >> 2): the A operand of 32-deep k-step s for output rows
//        16w..16w+15 of W M0, one 16-byte load a lane (value e reads state
//        row 16kb + 4g4 + (e & 3))
//   UA [pair 4][w 4][l][8]      = U~[16w + 4g4 + (e & 3)][16 (2 pair + (e >> 2)) + l16]
//        (accumulator layout; the two tiles of a sweep workgroup's pair side by
//        side, one 16-byte load a lane)
//   P  [w 4][ks 2][l][8]        P[16w + l16][32ks + 4g4 + (e & 3) + 16 (e >> 2)],
//        the A operands of P U in the permuted k order (below)
// The A operands of q^ M0 and the k^ of the update are the key head's, in its
// fragment block (qk_kernel).  Rows past the chunk's end are zero in every array.
constexpr int kOffW = 0, kOffUA = 8192, kOffP = 16384;
constexpr int kBlockElems = 20480;
// The gates of a chunk-head (fp32): [0] e^{gamma_L}, [4 + t] e^{gamma_t},
// [68 + t] e^{gamma_L - gamma_t}; zero past the chunk's end.
constexpr int kGv = 132, kGvEg = 4, kGvEk = 68;
// Word 3 of a raw buffer resource on gfx9-family chips (gfx950 included):
// 32-bit data format, no swizzle; accesses past num_records are dropped.
constexpr int kBufferDword3 = 0x00020000;
constexpr int kNonTemporal = 2;   // cache-policy operand of a buffer store: nt
constexpr int kDppSwapPairs = 0xB1;   // DPP quad_perm(1, 0, 3, 2): lanes 2m and 2m + 1 trade
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct Ctx {
    PrefillArgs P;
    int r;                      // value heads per key head
    int nc_total;               // chunk blocks in the workspace
    uint16_t *blk;
    float *gv;                  // per (chunk, value head): the gates the sweep scales by
    uint4 *frag;                // per (chunk, key head): q^ / k^ fragments (qk_kernel)
};

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

// The prompt and in-prompt chunk of dense chunk index cid (chunks numbered
// prompt after prompt).  False if cid is past the last chunk or the layout
// breaks the rules at or before its prompt (the same prompts prompt_chunks
// refuses).
__device__ bool chunk_at(const Ctx &X, int cid, int &p, int &c, int &s0, int &s1)
{
    const int T = X.P.total_rows;
    int base = 0;
    int prev = X.P.seq_start[0];
    if (prev < 0) return false;
    for (int q = 0; q < X.P.n_seqs; ++q) {
        const int a = X.P.seq_start[q], b = X.P.seq_start[q + 1];
        if (a != prev || b < a || b > T || b - a > X.P.max_len) return false;
        prev = b;
        const int nq = (b - a + kChunk - 1) / kChunk;
        if (cid < base + nq) {
            if (base + nq > X.nc_total) return false;
            p = q;
            c = cid - base;
            s0 = a;
            s1 = b;
            return true;
        }
        base += nq;
    }
    return false;
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(uint16_t *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }
__device__ __forceinline__ bf8v as_bf8(uint4 v) { return __builtin_bit_cast(bf8v, v); }

// bf16 value e (0..7) of a 16-byte vector, as fp32
__device__ __forceinline__ float bfe(const uint4 &u, int e)
{
    const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
}

__device__ __forceinline__ f4v mfma_bf16(uint4 a, uint4 b, f4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(a), as_bf8(b), c, 0, 0, 0);
}

// SiLU on the hardware's approximate exp2 and reciprocal (about 1 ulp each,
// no IEEE division sequence): every SiLU value of this pass is rounded to a
// bf16 matrix operand right after, 2^16 times coarser.
__device__ __forceinline__ float silu_fast(float y)
{
    return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * y));
}

// ---------------------------------------------------------------- intra
// T = (I + A)^-1 for the strictly lower-triangular 64 x 64 A, by 16 x 16
// blocks: the diagonal blocks B_i = (I + A_ii)^-1 by forward substitution,
// then T_ij = -B_i sum_{k=j}^{i-1} A_ik T_kj (i > j) on fp32 MFMA, one
// diagonal distance after the other.  An holds -A in fp32, 64 x 64; its
// strictly upper blocks are free and keep the fp32 T blocks later stages read
// (B_i over A_ii once that is used, T_10 in block (0,1), T_21 in (1,2), T_20
// in (0,2)).
// An's rows are AS = 68 floats apart (272 B, 4 banks on): a block operand
// read takes 16 rows at one column, which 256-byte rows put on the same
// banks (341 vs 346 us a 4-prompt pass, bit for bit the same).
constexpr int AS = 68;

// z += X Y for fp32 16 x 16 blocks X = An block (xi, xj), Y = An block (yi, yj)
__device__ __forceinline__ f4v mm_blocks(const float *An, int xi, int xj, int yi, int yj, f4v z, int l16, int g4)
{
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(An[(16 * xi + l16) * AS + 16 * xj + 4 * kk + g4],
                                                 An[(16 * yi + 4 * kk + g4) * AS + 16 * yj + l16], z, 0, 0, 0);
    return z;
}

// -B_i S for S held in the accumulator layout (register kk of lane l is
// S[4 g4 + kk][l16]), B_i = An block (i, i)
__device__ __forceinline__ f4v neg_diag_times(const float *An, int i, f4v s, int l16, int g4)
{
    f4v z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(-An[(16 * i + l16) * AS + 16 * i + 4 * g4 + kk], s[kk], z, 0, 0, 0);
    return z;
}

constexpr int SB = 72;   // bf16 row stride of the [.][64] LDS arrays (144 B: rows 4 banks apart)

// LDS of an intra workgroup (bytes): 47 KiB, three workgroups a CU
constexpr int kIntraAn = 0;                        // fp32 [64][AS]: -A, and T blocks later stages read
constexpr int kIntraPb = 64 * AS * 4;              // bf16 [64][SB]  P
constexpr int kIntraT1 = kIntraPb + 64 * SB * 2;   // bf16 [64][SB]  T' = T diag(beta e^gamma)
constexpr int kIntraT2 = kIntraT1 + 64 * SB * 2;   // bf16 [64][SB]  T'' = T diag(beta)
constexpr int kIntraVec = kIntraT2 + 64 * SB * 2;  // fp32 [4][64]   gamma, beta, e^gamma, e^{gamma_L - gamma}
constexpr int kIntraW = kIntraVec + 4 * 64 * 4;      // fp32 [128][4]  the value head's conv weights
constexpr int kIntraLds = kIntraW + D * 4 * 4;
constexpr int KSB = 136;   // bf16 row stride of the staged k^ / q^ rows (272 B: rows 4 banks apart)
static_assert(2 * 64 * KSB * 2 <= kIntraVec, "staged k^ and q^ fit below the gate vectors");

// Operands with a permuted k order.  A bf16 MFMA k-step ks reads, in lane
// group g4, the 8 contraction indices s = 32 ks + 4 g4 + {0..3} and
// s = 32 ks + 16 + 4 g4 + {0..3}: exactly the rows that the accumulator
// registers of the 16x16 blocks 2 ks and 2 ks + 1 hold in that lane group.
// A and B of one product use the same order, so an accumulator block pair
// feeds the next product straight from registers.
__device__ __forceinline__ uint4 pack_perm(f4v lo, f4v hi)
{
    return make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
}
// the same 8 indices of a bf16 LDS row
__device__ __forceinline__ uint4 lds_perm(const uint16_t *row, int ks, int g4)
{
    const uint2 lo = *reinterpret_cast<const uint2 *>(row + 32 * ks + 4 * g4);
    const uint2 hi = *reinterpret_cast<const uint2 *>(row + 32 * ks + 16 + 4 * g4);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
// B operand of X[16 rows][32 cols] times this = X[., 16 hb .. 16 hb + 16): a
// bf16 0/1 selection.  The product, exact, leaves register i of lane
// (l16, g4) holding X[4 g4 + i][16 hb + l16]: a transpose of the loaded rows.
__device__ __forceinline__ uint4 select_cols(int hb, int l16, int g4)
{
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int k0 = 8 * g4 + 2 * p;
        w[p] = ((k0 == 16 * hb + l16) ? 0x3F80u : 0u) | ((k0 + 1 == 16 * hb + l16) ? 0x3F800000u : 0u);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------- qk
// Per (chunk, key head): what the r value heads of a key head share, formed
// once.  The causal conv + SiLU of the chunk's q and k channels straight from
// the packed rows, their L2 norms (q also times dk^-1/2), K K^T and Q K^T on
// bf16 MFMA, and the fragments of k^ and q^ that the per-value-head kernel's
// products take.  Each wave leaves 16 uint4 a lane in the unit's fragment
// block, [wave 4][j 16][lane 64], in the registers and lane order that the
// per-value-head kernel's wave of the same index reads them:
//   j 0..3    K K^T block (w >> 1, w & 1), accumulator registers 4j .. 4j + 3
//   j 4..7    Q K^T block, the same way
//   j 8..11   kp[hb][ks] (j = 8 + 2 hb + ks): the transposed k^ fragments,
//             k^[32 ks + 4 g4 + (e & 3) + 16 (e >> 2)][32 w + 16 hb + l16]
//   j 12..15  q^[16 w + l16][16 kb + 4 g4 .. + 3] for kb = 2 (j - 12) (low
//             half) and kb + 1 (high half): the sweep's A operands of q^ M0
// The sweep's wave w reads the fragments k^ (j 8..11, the k^ of its state
// update) and q^ of wave w.
constexpr int kFragS = 0, kFragQK = 4, kFragKp = 8, kFragQ = 12, kFragVec4 = 16;
constexpr int kQkLds = 2 * 64 * KSB * 2;   // the staged k^ and q^ rows

__global__ void __launch_bounds__(256, 4) qk_kernel(const Ctx X)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int l32 = lane & 31, hh = lane >> 5;
    const int hk = X.P.hk;
    // workgroup i = unit i runs on XCD i % 8, where the per-value-head
    // workgroups of the same unit run and read its fragments
    const int unit = blockIdx.x;
    if (unit >= X.nc_total * hk) return;
    const int cid = unit / hk, kh = unit - cid * hk;
    int pidx, c, s0, s1;
    if (!chunk_at(X, cid, pidx, c, s0, s1)) return;
    const int r0 = s0 + c * kChunk;
    const int L = min(kChunk, s1 - r0);

    const int C = X.P.C, nq = hk * D;
    const uint16_t *tail = X.P.conv_tail + (size_t)pidx * 3 * C;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    // packed row u (>= r0 - 3) of channel group ch: the prompt's own row, or
    // row 3 + u - s0 of its conv tail before the prompt's first row
    auto raw_row = [&](int ch, int u) {
        return ld16(u >= s0 ? X.P.qkv + (size_t)u * C + ch : tail + (size_t)(3 + u - s0) * C + ch);
    };

    // ---- the chunk's k^ and q^ rows, staged in LDS.  Thread (which, c8) of 32 walks 8 consecutive
    // rows of 8 channels: the window's 11 raw rows requested together, then per
    // row causal conv + SiLU and the L2 norm over the 16 lanes of the head.
    // Rows past the chunk's end are zero (their raw rows are clamped to the
    // chunk's last row and never used).
    uint16_t *Ks = reinterpret_cast<uint16_t *>(lds);              // [64][KSB] k^
    uint16_t *Qs = Ks + 64 * KSB;                                  // [64][KSB] q^ (scaled)
    {
        const int which = (tid >> 4) & 1;                 // 0: k, 1: q
        const int c8 = (tid & 15) * 8, t0 = 8 * (tid >> 5);
        const int ch = (which ? 0 : nq) + kh * D + c8;
        float w[8][4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float4 wv = *reinterpret_cast<const float4 *>(X.P.conv_w + (size_t)(ch + e) * 4);
            w[e][0] = wv.x; w[e][1] = wv.y; w[e][2] = wv.z; w[e][3] = wv.w;
        }
        uint4 x[11];   // raw rows t0 - 3 .. t0 + 7 of the chunk
#pragma unroll
        for (int k = 0; k < 11; ++k) x[k] = raw_row(ch, min(r0 + t0 + k - 3, r0 + L - 1));
        const float qscale = which ? 1.0f / sqrtf((float)D) : 1.0f;
        uint16_t *dst = (which ? Qs : Ks) + c8;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float a[8];
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float y = w[e][0] * bfe(x[k], e);
                y = fmaf(w[e][1], bfe(x[k + 1], e), y);
                y = fmaf(w[e][2], bfe(x[k + 2], e), y);
                y = fmaf(w[e][3], bfe(x[k + 3], e), y);
                a[e] = silu_fast(y);
                ss = fmaf(a[e], a[e], ss);
            }
            ss = sum_row16(ss);   // over the 16 lanes of the head
            const float sc = __builtin_amdgcn_rsqf(ss + 1e-6f) * qscale;   // approximate 1/sqrt, as SiLU
            const uint4 o = make_uint4(pack2(a[0] * sc, a[1] * sc), pack2(a[2] * sc, a[3] * sc),
                                       pack2(a[4] * sc, a[5] * sc), pack2(a[6] * sc, a[7] * sc));
            st16(dst + (t0 + k) * KSB, t0 + k < L ? o : z4);
        }
    }

    lds_barrier();   // k^, q^ staged

    // ---- K K^T and Q K^T, wave w: the 32 x 32 block (w >> 1, w & 1); the
    // transposed fragments of k^, packed in the permuted k order: kp[hb][ks]
    // element j holds k^[32 ks + 4 g4 + (j & 3) + 16 (j >> 2)][32 w + 16 hb + l16]
    f16v S = {}, QK = {};
    {
        const int ra = 32 * (wave >> 1) + l32, rb = 32 * (wave & 1) + l32;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const int ko = 16 * ks + 8 * hh;
            const uint4 kb = ld16(Ks + rb * KSB + ko);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(ld16(Ks + ra * KSB + ko)), as_bf8(kb), S, 0, 0, 0);
            QK = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(ld16(Qs + ra * KSB + ko)), as_bf8(kb), QK, 0, 0, 0);
        }
    }
    uint4 kp[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const uint4 sel = select_cols(hb, l16, g4);
        const f4v z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            kp[hb][ks] = pack_perm(mfma_bf16(ld16(Ks + (32 * ks + l16) * KSB + 32 * wave + 8 * g4), sel, z),
                                   mfma_bf16(ld16(Ks + (32 * ks + 16 + l16) * KSB + 32 * wave + 8 * g4), sel, z));
    }

    // this wave's fragments, 1 KB contiguous a store
    uint4 *fr = X.frag + ((size_t)unit * 4 + wave) * kFragVec4 * 64 + lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        fr[(kFragS + j) * 64] = make_uint4(__float_as_uint(S[4 * j]), __float_as_uint(S[4 * j + 1]),
                                           __float_as_uint(S[4 * j + 2]), __float_as_uint(S[4 * j + 3]));
        fr[(kFragQK + j) * 64] = make_uint4(__float_as_uint(QK[4 * j]), __float_as_uint(QK[4 * j + 1]),
                                            __float_as_uint(QK[4 * j + 2]), __float_as_uint(QK[4 * j + 3]));
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) fr[(kFragKp + 2 * hb + ks) * 64] = kp[hb][ks];
#pragma unroll
    for (int kp2 = 0; kp2 < 4; ++kp2) {
        const uint16_t *q0 = Qs + (16 * wave + l16) * KSB + 32 * kp2 + 4 * g4;
        const uint2 lo = *reinterpret_cast<const uint2 *>(q0);
        const uint2 hi = *reinterpret_cast<const uint2 *>(q0 + 16);
        fr[(kFragQ + kp2) * 64] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
}

__global__ void __launch_bounds__(256, 3) intra_kernel(const Ctx X)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int l32 = lane & 31, hh = lane >> 5;
    // workgroup i runs on XCD i % 8.  The r value heads of one (chunk, key
    // head), which read the same fragments and q and k rows, are consecutive
    // workgroups of one XCD (the XCD where qk_kernel formed the fragments).
    const int r = X.r, hk = X.P.hk;
    const int xcd = blockIdx.x & 7, qi = blockIdx.x >> 3;
    const int unit = (qi / r) * 8 + xcd;              // (chunk, key head)
    if (unit >= X.nc_total * hk) return;
    const int cid = unit / hk, kh = unit - cid * hk;
    const int h = kh * r + (qi - (qi / r) * r);
    int pidx, c, s0, s1;
    if (!chunk_at(X, cid, pidx, c, s0, s1)) return;
    const int r0 = s0 + c * kChunk;
    const int L = min(kChunk, s1 - r0);
    const int hv = X.P.hv;
    const size_t cidh = (size_t)cid * hv + h;
    uint16_t *blk = X.blk + cidh * kBlockElems;
    // the chunk's gate inputs (wave 0 scans them first), requested before the
    // fragments so that their wait does not include the fragments'; rows past
    // the chunk's end read its last row (not used)
    const size_t go = (size_t)min(r0 + lane, r0 + L - 1) * X.P.hv + h;
    const float a_in = bf16f(X.P.a[go]), b_in = bf16f(X.P.b[go]);
    // this wave's fragments of the key head's k^ and q^ (qk_kernel)
    const uint4 *fr = X.frag + ((size_t)unit * 4 + wave) * kFragVec4 * 64 + lane;
    f16v S, QK;
    uint4 kp[2][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 sv = fr[(kFragS + j) * 64], qk = fr[(kFragQK + j) * 64];
        S[4 * j] = __uint_as_float(sv.x);
        S[4 * j + 1] = __uint_as_float(sv.y);
        S[4 * j + 2] = __uint_as_float(sv.z);
        S[4 * j + 3] = __uint_as_float(sv.w);
        QK[4 * j] = __uint_as_float(qk.x);
        QK[4 * j + 1] = __uint_as_float(qk.y);
        QK[4 * j + 2] = __uint_as_float(qk.z);
        QK[4 * j + 3] = __uint_as_float(qk.w);
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) kp[hb][ks] = fr[(kFragKp + 2 * hb + ks) * 64];

    float *An = reinterpret_cast<float *>(lds + kIntraAn);
    uint16_t *Pb = reinterpret_cast<uint16_t *>(lds + kIntraPb);
    uint16_t *T1 = reinterpret_cast<uint16_t *>(lds + kIntraT1);
    uint16_t *T2 = reinterpret_cast<uint16_t *>(lds + kIntraT2);
    float *gam = reinterpret_cast<float *>(lds + kIntraVec);
    float *bet = gam + 64, *eg = bet + 64;

    const int C = X.P.C, nq = hk * D;
    const uint16_t *tail = X.P.conv_tail + (size_t)pidx * 3 * C;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    // packed row u (>= r0 - 3) of channel group ch: the prompt's own row, or
    // row 3 + u - s0 of its conv tail before the prompt's first row
    auto raw_row = [&](int ch, int u) {
        return ld16(u >= s0 ? X.P.qkv + (size_t)u * C + ch : tail + (size_t)(3 + u - s0) * C + ch);
    };

    // the value head's conv weights, one 16-byte piece a thread of waves 1 and
    // 2, for the v conv after the solve (one load a thread instead of eight)
    float4 *wl = reinterpret_cast<float4 *>(lds + kIntraW);
    if (tid >= 64 && tid < 64 + D)
        wl[tid - 64] = *reinterpret_cast<const float4 *>(X.P.conv_w + (size_t)(2 * nq + h * D + tid - 64) * 4);
    // ---- gates: gamma (inclusive in-chunk scan of log alpha), beta and the decays
    if (wave == 0) {
        float gl = lane < L ? log_decay(a_in, X.P.a_log[h], X.P.dt_bias[h]) : 0.0f;
        const float bl = lane < L ? sigmoid_f(b_in) : 0.0f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float up = __shfl_up(gl, d);
            if (lane >= d) gl += up;
        }
        const float gL = __shfl(gl, L - 1);
        const float egl = lane < L ? __expf(gl) : 0.0f;
        gam[lane] = gl;
        bet[lane] = bl;
        eg[lane] = egl;
        // the sweep's scales: e^{gamma_L} of the chunk, e^gamma of each
        // output row, e^{gamma_L - gamma} of each row's delta
        float *gv = X.gv + cidh * kGv;
        if (lane == 0) gv[0] = __expf(gL);
        gv[kGvEg + lane] = egl;
        gv[kGvEk + lane] = lane < L ? __expf(gL - gl) : 0.0f;
    }

    lds_barrier();   // gamma, beta visible

    // -A (strictly lower, fp32) and P (lower with diagonal, bf16)
    {
        const int bi = wave >> 1, bj = wave & 1;
        const int s = 32 * bj + l32;
        const float gs = gam[s];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 32 * bi + 8 * (i >> 2) + 4 * hh + (i & 3);
            // branch-free: the decay's argument is selected (e^-inf = +0,
            // as the zero it stands for) and every read is made, so the
            // compiler batches the reads instead of branching sixteen times
            // around each (339 vs 344 us a pass, bit for bit the same)
            const bool live = s <= t && t < L;
            const float gt = gam[t], bt = bet[t];
            const float dec = __expf(live ? gt - gs : -__builtin_inff());
            const float a = -bt * dec * S[i];
            An[t * AS + s] = (live && s < t) ? a : 0.0f;
            Pb[t * SB + s] = f2bf(dec * QK[i]);
        }
    }
    lds_barrier();

    // ---- T = (I + A)^-1 by 16 x 16 blocks, stored scaled by columns as
    // T' = T diag(beta e^gamma) and T'' = T diag(beta) (bf16).  Stage 1: wave w
    // inverts diagonal block w (every lane group computes column l16; group
    // g4 stores rows 4 g4 .. 4 g4 + 3)
    {
        const int j = l16, w = wave;
        float Tc[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = (t == j) ? 1.0f : 0.0f;
            const float *row = An + (16 * w + t) * AS + 16 * w;
#pragma unroll
            for (int s = 0; s < t; ++s) acc = fmaf(row[s], Tc[s], acc);
            Tc[t] = acc;
            // one row's reads at a time: hoisting all 120 would hold them in registers
            __builtin_amdgcn_sched_barrier(0);
        }
        const float b1 = bet[16 * w + j] * eg[16 * w + j], b2 = bet[16 * w + j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = g4 == 0 ? Tc[i] : g4 == 1 ? Tc[4 + i] : g4 == 2 ? Tc[8 + i] : Tc[12 + i];
            const int t = 16 * w + 4 * g4 + i;
            An[t * AS + 16 * w + j] = v;
            T1[t * SB + 16 * w + j] = f2bf(v * b1);
            T2[t * SB + 16 * w + j] = f2bf(v * b2);
            for (int cb = w + 1; cb < 4; ++cb) {
                T1[t * SB + 16 * cb + j] = 0;
                T2[t * SB + 16 * cb + j] = 0;
            }
        }
    }
    lds_barrier();
    // store a finished 16 x 16 block (i, j) of T, accumulator layout, scaled
    auto put_t = [&](int i, int jb, const f4v &z) {
        const float b1 = bet[16 * jb + l16] * eg[16 * jb + l16], b2 = bet[16 * jb + l16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * i + 4 * g4 + r;
            T1[t * SB + 16 * jb + l16] = f2bf(z[r] * b1);
            T2[t * SB + 16 * jb + l16] = f2bf(z[r] * b2);
        }
    };
    // v's raw rows for the conv below, thread (channel group vcg, rows
    // vt0 - 3 .. vt0 + 3 of the chunk), requested here so that the rest of
    // the solve covers their wait (362 -> 348 us a 4-prompt pass, bit for bit
    // the same); during the diagonal blocks' substitution they would not fit
    // in the registers beside it
    const int vcg = tid & 15, vt0 = 4 * (tid >> 4);
    uint4 vx[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) vx[k] = raw_row(2 * nq + h * D + 8 * vcg, min(r0 + vt0 + k - 3, r0 + L - 1));
    // Stage 2: T_{i,i-1} = -B_i A_{i,i-1} B_{i-1}, wave i (An holds -A)
    if (wave >= 1) {
        const int i = wave;
        f4v x = {0.f, 0.f, 0.f, 0.f};
        x = mm_blocks(An, i, i - 1, i - 1, i - 1, x, l16, g4);   // -A_{i,i-1} B_{i-1}
        const f4v z = -neg_diag_times(An, i, x, l16, g4);
        put_t(i, i - 1, z);
        if (i < 3) {
#pragma unroll
            for (int r = 0; r < 4; ++r) An[(16 * (i - 1) + 4 * g4 + r) * AS + 16 * i + l16] = z[r];   // T_10 -> (0,1), T_21 -> (1,2)
        }
    }
    lds_barrier();
    // Stage 3: T_{i,i-2} = -B_i (A_{i,i-2} B_{i-2} + A_{i,i-1} T_{i-1,i-2}), waves 2 and 3
    if (wave >= 2) {
        const int i = wave;
        f4v x = {0.f, 0.f, 0.f, 0.f};
        x = mm_blocks(An, i, i - 2, i - 2, i - 2, x, l16, g4);
        x = mm_blocks(An, i, i - 1, i - 2, i - 1, x, l16, g4);   // T_{i-1,i-2} is kept in block (i-2, i-1)
        const f4v z = -neg_diag_times(An, i, x, l16, g4);
        put_t(i, i - 2, z);
        if (i == 2) {
#pragma unroll
            for (int r = 0; r < 4; ++r) An[(4 * g4 + r) * AS + 32 + l16] = z[r];   // T_20 -> (0,2)
        }
    }
    lds_barrier();
    // Stage 4: T_30 = -B_3 (A_30 B_0 + A_31 T_10 + A_32 T_20), wave 3
    if (wave == 3) {
        f4v x = {0.f, 0.f, 0.f, 0.f};
        x = mm_blocks(An, 3, 0, 0, 0, x, l16, g4);
        x = mm_blocks(An, 3, 1, 0, 1, x, l16, g4);
        x = mm_blocks(An, 3, 2, 0, 2, x, l16, g4);
        put_t(3, 0, -neg_diag_times(An, 3, x, l16, g4));
    }
    lds_barrier();

    // ---- v of value head h: causal conv + SiLU from the raw rows (in vx since
    // the solve's second stage), staged as bf16 in the space of -A, which the
    // solve no longer reads.  Vs row t holds 16 groups of 8 channels, group c
    // at position c ^ (t & 15), so that both the row-wise writes and the
    // column-wise reads below meet 16 distinct banks.  Thread (c, rows
    // 4 j .. 4 j + 3) holds the 7 raw rows it needs.
    uint16_t *Vs = reinterpret_cast<uint16_t *>(lds + kIntraAn);   // [64][128]
    {
        const int cg = vcg, t0 = vt0;
        const uint4 *x = vx;   // raw rows t0 - 3 .. t0 + 3 of the chunk
        float w[8][4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float4 wv = wl[8 * cg + e];
            w[e][0] = wv.x; w[e][1] = wv.y; w[e][2] = wv.z; w[e][3] = wv.w;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = t0 + k;
            float a[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float y = w[e][0] * bfe(x[k], e);
                y = fmaf(w[e][1], bfe(x[k + 1], e), y);
                y = fmaf(w[e][2], bfe(x[k + 2], e), y);
                y = fmaf(w[e][3], bfe(x[k + 3], e), y);
                a[e] = silu_fast(y);
            }
            const uint4 o = make_uint4(pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(a[4], a[5]), pack2(a[6], a[7]));
            st16(Vs + t * D + 8 * (cg ^ (t & 15)), t < L ? o : z4);
        }
    }
    lds_barrier();
    // v rows 16 mt + l16, channels [32w + 8 g4, + 8)
    uint4 vr[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) vr[mt] = ld16(Vs + (16 * mt + l16) * D + 8 * ((4 * wave + g4) ^ l16));
    // ---- the products, wave w on key column blocks kb = 2w + hb and value
    // tiles 2w + hb (hb = 0, 1), with the permuted k order throughout:
    //  W^T = k^T T'^T  (kb, mt) -> the sweep's W
    //  U~  = T'' v     (mt, tile) -> the sweep's UA
    uint4 vp[2][2];   // v fragments, packed like kp
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const uint4 sel = select_cols(hb, l16, g4);
        const f4v z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            vp[hb][ks] = pack_perm(mfma_bf16(vr[2 * ks], sel, z), mfma_bf16(vr[2 * ks + 1], sel, z));
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        uint4 t1[2], t2[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            t1[ks] = lds_perm(T1 + (16 * mt + l16) * SB, ks, g4);
            t2[ks] = lds_perm(T2 + (16 * mt + l16) * SB, ks, g4);
        }
        f4v wt[2], u[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            wt[hb] = f4v{0.f, 0.f, 0.f, 0.f};
            u[hb] = wt[hb];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                wt[hb] = mfma_bf16(kp[hb][ks], t1[ks], wt[hb]);
                u[hb] = mfma_bf16(t2[ks], vp[hb][ks], u[hb]);
            }
        }
        // wt[hb]: lane holds W[16 mt + l16][16 kb + 4 g4 + i], u[hb]: U~[16 mt + 4 g4 + i][16 kb + l16]
        // for kb = 2 wave + hb: the two halves of one 16-byte piece each
        *reinterpret_cast<uint4 *>(blk + kOffW + ((mt * 4 + wave) * 64 + lane) * 8) =
            make_uint4(pack2(wt[0][0], wt[0][1]), pack2(wt[0][2], wt[0][3]), pack2(wt[1][0], wt[1][1]), pack2(wt[1][2], wt[1][3]));
        *reinterpret_cast<uint4 *>(blk + kOffUA + ((wave * 4 + mt) * 64 + lane) * 8) =
            make_uint4(pack2(u[0][0], u[0][1]), pack2(u[0][2], u[0][3]), pack2(u[1][0], u[1][1]), pack2(u[1][2], u[1][3]));
        // bound how far the scheduler hoists the next block's LDS reads
        __builtin_amdgcn_sched_barrier(0);
    }
    //  P rows 16 w .. 16 w + 15 -> the sweep's P, in the permuted k order
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
        st16(blk + kOffP + ((wave * 2 + ks) * 64 + lane) * 8, lds_perm(Pb + (16 * wave + l16) * SB, ks, g4));
}

// ---------------------------------------------------------------- sweep
// The state contractions of the sweep (W M0, q^ M0 and the update k^T U')
// pair a bf16 A operand (W, q^, k^ as the per-chunk kernels left them) with
// an fp32 B operand (M0, or U' = e^{gamma_L - gamma} U).  An fp32 value x is
// the exact sum of three bf16 values: t0 = x with its low 16 bits cleared,
// t1 the same of x - t0, t2 = x - t0 - t1 (at most 8 significant bits, so a
// bf16 exactly).  Each contraction runs as three bf16 MFMAs, one a term:
// every product of a term with a bf16 operand is exact in fp32, and their
// sum is a x up to the fp32 rounding of the accumulation, as in an fp32 MFMA
// of the same operands (48 matrix-core cycles a 32-deep k-step instead of
// 256).  The wave that holds a value splits it, once a chunk.
//
// A workgroup takes two adjacent 16-column tiles of a head (32 state
// columns), so that the chunk's W, q^, k^ and P operands, which every tile of
// the head reads whole, are requested once for both (the 4-prompt pass: 464
// -> 398 us against one tile a workgroup).  Wave w keeps state rows
// [32 w, 32 w + 32) x 32 columns (four 16 x 16 accumulators) and takes
// output rows [16 w, 16 w + 16) of both tiles.
//
// LDS of a sweep workgroup, uint4 a lane (every access 16 or 8 bytes a lane,
// lanes consecutive), tile t of the pair:
//   Mb [3 terms][4 k-steps s][2 tiles][64 lanes]  the B operand of k-step s
//        of W M0 and q^ M0: M0 rows 32 s + 4 g4 + {0..3} and
//        32 s + 16 + 4 g4 + {0..3}, column 16 t + l16 of the pair -- the two
//        accumulator blocks of wave s, as they sit
//   Ub [2 k-steps][2 tiles][64]  U rounded to bf16 (nearest), the B operand
//        of P U: rows 32 ks + 4 g4 + {0..3} (wave 2 ks) and
//        32 ks + 16 + 4 g4 + {0..3} (wave 2 ks + 1)
//   Us [3 terms][2 k-steps][2 tiles][64]  the terms of U', the B operand of
//        the update, the same rows
constexpr int kSwMb = 0, kSwUb = 24 * 64, kSwUs = kSwUb + 4 * 64, kSwLds = kSwUs + 12 * 64;

__device__ __forceinline__ f4v ldg4(const float *p) { return *reinterpret_cast<const f4v *>(p); }
// the high halves of two words: bf16 (truncated) of two fp32 values
__device__ __forceinline__ uint32_t high2(uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x07060302u); }

// the three bf16 terms of four fp32 values, 4 bf16 (8 bytes) each
__device__ __forceinline__ void split4(f4v x, uint2 &t0, uint2 &t1, uint2 &t2)
{
    uint32_t a[4], b[4], c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = __float_as_uint(x[e]);
        const float r1 = x[e] - __uint_as_float(a[e] & 0xffff0000u);
        b[e] = __float_as_uint(r1);
        c[e] = __float_as_uint(r1 - __uint_as_float(b[e] & 0xffff0000u));
    }
    t0 = make_uint2(high2(a[0], a[1]), high2(a[2], a[3]));
    t1 = make_uint2(high2(b[0], b[1]), high2(b[2], b[3]));
    t2 = make_uint2(high2(c[0], c[1]), high2(c[2], c[3]));
}

// wave w's state blocks of both tiles into Mb, in their three terms
__device__ __forceinline__ void put_state(uint4 *sw, int wave, int lane, const f4v (&M)[2][2])
{
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        uint2 a0, a1, a2, b0, b1, b2;
        split4(M[t][0], a0, a1, a2);
        split4(M[t][1], b0, b1, b2);
        sw[kSwMb + ((0 * 4 + wave) * 2 + t) * 64 + lane] = make_uint4(a0.x, a0.y, b0.x, b0.y);
        sw[kSwMb + ((1 * 4 + wave) * 2 + t) * 64 + lane] = make_uint4(a1.x, a1.y, b1.x, b1.y);
        sw[kSwMb + ((2 * 4 + wave) * 2 + t) * 64 + lane] = make_uint4(a2.x, a2.y, b2.x, b2.y);
    }
}

__global__ void __launch_bounds__(256) sweep_kernel(const Ctx X)
{
    __shared__ uint4 sw[kSwLds];
    __shared__ int order[256];      // prompt of each length rank
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: operand bases stay scalar
    const int l16 = lane & 15, g4 = lane >> 4;
    const int hv = X.P.hv;
    // workgroup i runs on XCD i % 8: the 4 tile pairs of the r value heads of
    // one (prompt, key head) go to one XCD, where they share the key head's
    // fragments and each head's operand blocks in L2
    const int r = X.r, hk = X.P.hk;
    constexpr int NP = NTILE / 2;             // tile pairs of a head
    const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    const int tp = q & (NP - 1);
    const int gq = q / NP;                    // value-head slot on this XCD
    const int u = (gq / r) * 8 + xcd;         // (prompt rank, key head)
    if (u >= X.P.n_seqs * hk) return;
    const int rank = u / hk, h = (u - rank * hk) * r + (gq - (gq / r) * r);

    // prompts by decreasing length (ties by index): the longest chains start first
    const int n = X.P.n_seqs;
    int pidx = rank;
    if (n <= 256) {
        if (tid < n) {
            const int len = X.P.seq_start[tid + 1] - X.P.seq_start[tid];
            int rk = 0;
            for (int p = 0; p < n; ++p) {
                const int lp = X.P.seq_start[p + 1] - X.P.seq_start[p];
                rk += (lp > len) || (lp == len && p < tid);
            }
            order[rk] = tid;
        }
        lds_barrier();
        pidx = order[rank];
    }
    int s0, s1, cid0;
    if (!prompt_chunks(X, pidx, s0, s1, cid0)) return;
    const int nck = (s1 - s0 + kChunk - 1) / kChunk;
    if (nck == 0) return;
    const int col = 32 * tp + l16;            // tile t: column col + 16 t

    // this wave updates state rows [32 wave, 32 wave + 32): block b register i
    // is row 32 wave + 16 b + 4 g4 + i (the 16x16 accumulator layout)
    float *st = X.P.state + ((size_t)pidx * hv + h) * D * D + col;
    f4v M[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) M[t][b][i] = st[(size_t)(32 * wave + 16 * b + 4 * g4 + i) * D + 16 * t];
    put_state(sw, wave, lane, M);

    const size_t cstride = (size_t)hv * kBlockElems;
    const uint16_t *bp = X.blk + ((size_t)cid0 * hv + h) * kBlockElems;
    const uint16_t *pW = bp + kOffW + ((size_t)wave * 4 * 64 + lane) * 8;
    const uint16_t *pUA = bp + kOffUA + ((size_t)(tp * 4 + wave) * 64 + lane) * 8;
    const uint16_t *pP = bp + kOffP + ((size_t)wave * 2 * 64 + lane) * 8;
    // the key head's q^ and k^ fragments (qk_kernel), this wave's
    const int kh = h / X.r;
    const size_t fstride = (size_t)X.P.hk * 4 * kFragVec4 * 64;
    const uint4 *pF = X.frag + (((size_t)cid0 * X.P.hk + kh) * 4 + wave) * kFragVec4 * 64 + lane;
    // the gates: e^{gamma_L}, and this lane's rows' e^gamma and e^{gamma_L - gamma}
    const size_t gstride = (size_t)hv * kGv;
    const float *pG = X.gv + ((size_t)cid0 * hv + h) * kGv;
    const size_t orow = (size_t)hv * D;
    auto out_rsrc = [&](int c) {
        const int r0 = s0 + c * kChunk;
        const int L = min(kChunk, s1 - r0);
        return __builtin_amdgcn_make_buffer_rsrc(X.P.out + (size_t)r0 * orow, 0,
                                                 (int)((size_t)L * orow * sizeof(float)), kBufferDword3);
    };
    // this lane's output elements: rows 16 wave + 4 g4 + i of the chunk,
    // column col (+ 16 t) of head h
    int ooff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ooff[i] = (int)(((size_t)(16 * wave + 4 * g4 + i) * orow + (size_t)h * D + col) * 4);

    uint4 ww[4];
    uint4 wq[4], kt[4], pp[2];
    uint4 ua;          // U~ of this lane's rows: tile 0 in x, y; tile 1 in z, w
    float eL;
    f4v eg4, ek4;
    // first chunk's operands, requested in the order the loop requests the
    // next chunk's (W, q^; ua; P; k^, gates), so the memory-counter waits at
    // the loop head see one request order on both of its entries
#pragma unroll
    for (int s = 0; s < 4; ++s) ww[s] = ld16(pW + s * 512);
#pragma unroll
    for (int j = 0; j < 4; ++j) wq[j] = pF[(kFragQ + j) * 64];
    __builtin_amdgcn_sched_barrier(0);
    ua = ld16(pUA);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pp[ks] = ld16(pP + ks * 512);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) kt[j] = pF[(kFragKp + j) * 64];
    eL = pG[0];
    eg4 = ldg4(pG + kGvEg + 16 * wave + 4 * g4);
    ek4 = ldg4(pG + kGvEk + 16 * wave + 4 * g4);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();   // Mb complete

    // The loop is branch-free, so the compiler's memory-counter waits track
    // each operand exactly: each operand of chunk c + 1 is requested right
    // after its last use in chunk c (the last chunk requests its own again),
    // and output rows past a chunk's end are dropped by the buffer range check.
    for (int c = 0; c < nck; ++c) {
        const int cn = min(c + 1, nck - 1);
        const size_t nx = (size_t)cn * cstride, nf = (size_t)cn * fstride, ng = (size_t)cn * gstride;

        // W M0 and (e^gamma q) M0 for rows [16 wave, 16 wave + 16) over all 128
        // state rows, tile after tile: four 32-deep k-steps, three terms each.
        // A tile's B operands are read from LDS together before its products
        // (read one k-step at a time, each wait stalls the matrix core).
        f4v aU[2], aO[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            aU[t] = f4v{0.f, 0.f, 0.f, 0.f};
            aO[t] = aU[t];
            uint4 mb[3][4];
#pragma unroll
            for (int tm = 0; tm < 3; ++tm)
#pragma unroll
                for (int s = 0; s < 4; ++s) mb[tm][s] = sw[kSwMb + ((tm * 4 + s) * 2 + t) * 64 + lane];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int tm = 0; tm < 3; ++tm) {
                    aU[t] = mfma_bf16(ww[s], mb[tm][s], aU[t]);
                    aO[t] = mfma_bf16(wq[s], mb[tm][s], aO[t]);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) ww[s] = ld16(pW + nx + s * 512);
#pragma unroll
        for (int j = 0; j < 4; ++j) wq[j] = pF[nf + (kFragQ + j) * 64];

        // U = U~ - W M0: to Ub rounded, U' = e^{gamma_L - gamma} U to Us in terms
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f4v U;
            const uint32_t u01 = t ? ua.z : ua.x, u23 = t ? ua.w : ua.y;
            U[0] = __uint_as_float(u01 << 16) - aU[t][0];
            U[1] = __uint_as_float(u01 & 0xffff0000u) - aU[t][1];
            U[2] = __uint_as_float(u23 << 16) - aU[t][2];
            U[3] = __uint_as_float(u23 & 0xffff0000u) - aU[t][3];
            uint2 *ub_mine = reinterpret_cast<uint2 *>(sw + kSwUb + ((wave >> 1) * 2 + t) * 64 + lane) + (wave & 1);
            uint2 *us_mine = reinterpret_cast<uint2 *>(sw + kSwUs + ((wave >> 1) * 2 + t) * 64 + lane) + (wave & 1);
            *ub_mine = make_uint2(pack2(U[0], U[1]), pack2(U[2], U[3]));
            uint2 t0, t1, t2;
            split4(U * ek4, t0, t1, t2);
            us_mine[0] = t0;
            us_mine[2 * 2 * 64 * 2] = t1;       // uint2 units: a term is 2 k-steps x 2 tiles x 64 lanes x 2 halves
            us_mine[2 * 2 * 2 * 64 * 2] = t2;
        }
        __builtin_amdgcn_sched_barrier(0);
        ua = ld16(pUA + nx);
        lds_barrier();   // Ub, Us complete; every wave is done reading Mb

        float ov[2][4];   // o of this lane's rows and columns, both tiles
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            uint4 ub[2], us[3][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) ub[ks] = sw[kSwUb + (ks * 2 + t) * 64 + lane];
#pragma unroll
            for (int tm = 0; tm < 3; ++tm)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) us[tm][ks] = sw[kSwUs + ((tm * 2 + ks) * 2 + t) * 64 + lane];
            __builtin_amdgcn_sched_barrier(0);
            // O = e^gamma (q^ M0) + P U: P U on bf16 MFMA (an in-chunk product)
            f4v pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) pu = mfma_bf16(pp[ks], ub[ks], pu);
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[t][i] = fmaf(eg4[i], aO[t][i], pu[i]);
            // M <- e^{gamma_L} M + k^T U' on this wave's rows of tile t
#pragma unroll
            for (int b = 0; b < 2; ++b) M[t][b] = M[t][b] * eL;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int tm = 0; tm < 3; ++tm)
#pragma unroll
                    for (int b = 0; b < 2; ++b) M[t][b] = mfma_bf16(kt[2 * b + ks], us[tm][ks], M[t][b]);
        }
        {
            // o leaves in 8-byte stores: lanes 2m and 2m + 1 trade one value a
            // row (a DPP swap), so that the even lane holds tile 0's columns
            // 2m, 2m + 1 and the odd one tile 1's (8 stores a wave and chunk
            // became 4: 398 -> 384 us).  Rows past the chunk's end are dropped
            // by the buffer range check.  The stores are non-temporal: nothing
            // in the pass reads o, and the operand blocks the other tiles of
            // the head still read stay in L2.
            const __amdgpu_buffer_rsrc_t orsrc = out_rsrc(c);
            const bool odd = lane & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float give = odd ? ov[0][i] : ov[1][i];
                const float got = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(give), kDppSwapPairs, 0xF, 0xF, false));
                const u32x2 v = {__float_as_uint(odd ? got : ov[0][i]), __float_as_uint(odd ? ov[1][i] : got)};
                __builtin_amdgcn_raw_buffer_store_b64(v, orsrc, ooff[i] + (odd ? 15 * 4 : 0), 0, kNonTemporal);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) pp[ks] = ld16(pP + nx + ks * 512);
#pragma unroll
        for (int j = 0; j < 4; ++j) kt[j] = pF[nf + (kFragKp + j) * 64];
        eL = pG[ng];
        eg4 = ldg4(pG + ng + kGvEg + 16 * wave + 4 * g4);
        ek4 = ldg4(pG + ng + kGvEk + 16 * wave + 4 * g4);
        put_state(sw, wave, lane, M);
        lds_barrier();   // Mb complete; every wave is done reading Ub and Us
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) st[(size_t)(32 * wave + 16 * b + 4 * g4 + i) * D + 16 * t] = M[t][b][i];

    // the prompt's conv tail: its last three raw rows, continuing into the old
    // tail when the prompt is shorter.  Every read of the old tail (the
    // per-chunk kernel's) has finished: this launch follows it on the stream.
    // The (head, tile pair) workgroups of the prompt split the channel groups;
    // one thread reads all three old rows of a group before it writes any.
    {
        const int C = X.P.C, len = s1 - s0;
        uint16_t *tl = X.P.conv_tail + (size_t)pidx * 3 * C;
        const int units = C / 8, part = hv * NP;
        for (int v = h * NP + tp + part * tid; v < units; v += part * 256) {
            uint4 nt[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int m = len - 3 + j;   // local row of new tail row j
                nt[j] = ld16(m >= 0 ? X.P.qkv + (size_t)(s0 + m) * C + 8 * v : tl + (size_t)(m + 3) * C + 8 * v);
            }
#pragma unroll
            for (int j = 0; j < 3; ++j) st16(tl + (size_t)j * C + 8 * v, nt[j]);
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

PrefillLayout prefill_layout(int hk, int hv, int dk, int dv, int n_seqs, int T)
{
    PrefillLayout Lo = {};
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
    // each prompt adds at most one partial chunk to floor(T / 64) whole ones
    Lo.max_chunks_total = T / kChunk + n_seqs;
    const size_t nc = (size_t)Lo.max_chunks_total;
    Lo.blk = take(nc * hv * kBlockElems * 2);
    Lo.gv = take(nc * hv * kGv * 4);
    Lo.frag = take(nc * hk * 4 * kFragVec4 * 64 * sizeof(uint4));
    Lo.total = o;
    return Lo;
}

bool prefill_supported(int hk, int hv, int dk, int dv)
{
    return dk == D && dv == D && hk > 0 && hv % hk == 0 && hv / hk <= 8;
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
    X.nc_total = Lo.max_chunks_total;
    X.blk = reinterpret_cast<uint16_t *>(ws + Lo.blk);
    X.gv = reinterpret_cast<float *>(ws + Lo.gv);
    X.frag = reinterpret_cast<uint4 *>(ws + Lo.frag);

    static const hipError_t e_lds = hipFuncSetAttribute(reinterpret_cast<const void *>(intra_kernel),
                                                        hipFuncAttributeMaxDynamicSharedMemorySize, kIntraLds);
    if (e_lds != hipSuccess) return e_lds;


    const unsigned units = (unsigned)X.nc_total * P.hk;   // (chunk, key head) pairs
    hipLaunchKernelGGL(qk_kernel, dim3(units), dim3(256), kQkLds, stream, X);
    hipLaunchKernelGGL(intra_kernel, dim3(8 * X.r * ((units + 7) / 8)), dim3(256), kIntraLds, stream, X);
    const unsigned kunits = (unsigned)P.n_seqs * P.hk;   // (prompt, key head) pairs
    hipLaunchKernelGGL(sweep_kernel, dim3(8 * (NTILE / 2) * X.r * ((kunits + 7) / 8)), dim3(256), 0, stream, X);
    return hipGetLastError();
}

}  // namespace gdn
