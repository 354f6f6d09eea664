// Affine 4-bit in-projection of libgdn (gfx950): the mixer's inputs qkv, a
// and b from hidden rows x, y = x W^T, with W stored as 4-bit codes and a
// bf16 scale and bias per output feature and group of inputs
// (w = s * q + b; page "perf(qwen3_5 cuda): deliver the first token before
// drafting", the note on the MLX affine 4-bit checkpoint, whose projections
// run through affine-4 kernels; the format is MLX's affine quantisation).
//
// Each weight is expanded to bf16 (s * q + b in fp32, rounded to nearest
// even) right before it enters the matrix cores (v_mfma_f32_16x16x32_bf16
// in the small kernel, v_mfma_f32_32x32x16_bf16 in the large one), as MLX's
// own matrix kernels do; products accumulate in fp32 and the outputs are
// rounded to bf16.
//
// The small kernel takes inputs in chunks of 128.  Within a chunk, lane
// (l16, g4) of a wave owns inputs [32 g4, 32 g4 + 32): four consecutive code
// words, one 16-byte load, and in k-step s (0..3) it supplies inputs
// 32 g4 + 8 s .. + 8 of both operands (A: row l16 of x, B: feature l16 of W),
// so that every input meets its weight once.  Those 32 inputs lie in one
// group (group sizes 32, 64, 128): one scale and one bias serve the lane for
// the chunk.  The large kernel expands weights the same way, 16 or 32 inputs
// of one feature (a pair or a quad of code words) a thread, into LDS.
//
//   decode (rows <= 16, hidden <= 5120): a workgroup is one to three blocks
//          of 16 features x 16 rows; its 8 waves split the inputs and
//          request all their weights at once.
//   small  (rows <= 32): a workgroup is one or two blocks of 16 features x
//          16 or 32 rows; its 8 waves split the inputs.
//   large  a workgroup is 128 features x 128 or 256 rows on 32 x 32
//          matrix-core blocks; the chunk of x and the chunk of weights
//          (expanded once) are staged in LDS for its waves, and the output
//          tile leaves through LDS in whole rows where it lies inside qkv.
//          Launches with few tiles split the inputs between two groups of
//          waves in each workgroup.
//
// Weights come in a tiled layout, repacked once from MLX's by
// gdn_inproj_pack_affine4: features in blocks of 16 (the last padded with
// zero codes, scales and biases), per block and 128-input chunk one 1 KB piece
// [lane = 16 g4 + l16][4 words] holding words 16 c + 4 g4 .. + 3 of feature
// 16 block + l16, and scales and biases as [block][group][16].  So a wave's
// code words of a chunk are one contiguous 1 KB read, and 16 features' scales
// one 32-byte read.
#include "gdn_device.h"
#include "gdn_inproj.h"

namespace gdn {
namespace {

constexpr int kChunk = 128;

__device__ __forceinline__ uint4 ld16g(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ f4v mfma16x16x32(uint4 a, uint4 b, f4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, a), __builtin_bit_cast(bf8v, b), c,
                                                  0, 0, 0);
}

// The eight weights of one code word (code j in bits 4j..4j+3), s * q + b
// rounded to bf16, as a B operand in input order.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float s, float b)
{
    // even codes in the bytes of lo, odd codes in the bytes of hi: each code
    // then converts with one byte-to-float instruction (written out: the
    // compiler would extract each byte first)
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    float q[8], v[8];
    asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(q[0]) : "v"(lo));
    asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(q[2]) : "v"(lo));
    asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(q[4]) : "v"(lo));
    asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(q[6]) : "v"(lo));
    asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(q[1]) : "v"(hi));
    asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(q[3]) : "v"(hi));
    asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(q[5]) : "v"(hi));
    asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(q[7]) : "v"(hi));
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fmaf(s, q[j], b);
    return make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Output feature n of row r (both in range), to qkv, a or b.
__device__ __forceinline__ void put(const InprojArgs &A, int r, int n, float y)
{
    const uint16_t v = f2bf(y);
    if (n < A.channels)
        A.qkv[(size_t)r * A.channels + n] = v;
    else if (n < A.channels + A.hv)
        A.a[(size_t)r * A.hv + (n - A.channels)] = v;
    else
        A.b[(size_t)r * A.hv + (n - A.channels - A.hv)] = v;
}

// ---------------------------------------------------------------- small
// A workgroup is NF blocks of 16 features x 16 MS rows; its 8 waves take
// every 8th chunk (each wave's next chunk in flight while one computes) and
// add their partial sums in LDS in a fixed order.  A wave's code words of a
// chunk and block are one contiguous 1 KB piece of the tiled layout; its x
// pieces serve all NF blocks (two blocks halve the reads of x, which every
// workgroup reads whole).
template <int MS, int NF>
__global__ void __launch_bounds__(512) inproj_small_kernel(const InprojArgs A)
{
    constexpr int W = 8;
    __shared__ f4v red[W][NF * MS][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int features = A.channels + 2 * A.hv;
    const int blocks = (features + 15) / 16;
    const int nck = A.hidden / kChunk, ng = A.hidden / A.group;
    const int r0 = blockIdx.y * 16 * MS;
    // (past the last block, a workgroup's second block repeats the last one
    // and writes nothing)
    const uint32_t *wblk[NF];
    const uint16_t *sblk[NF], *bblk[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int nb = min((int)blockIdx.x * NF + f, blocks - 1);
        wblk[f] = A.wq + (size_t)nb * nck * 256 + 4 * lane;
        sblk[f] = A.scales + (size_t)nb * ng * 16 + l16;
        bblk[f] = A.biases + (size_t)nb * ng * 16 + l16;
    }
    const uint16_t *xrow[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) xrow[m] = A.x + (size_t)min(r0 + 16 * m + l16, A.rows - 1) * A.hidden + 32 * g4;

    f4v acc[NF][MS];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int m = 0; m < MS; ++m) acc[f][m] = f4v{0.f, 0.f, 0.f, 0.f};
    uint4 wv[NF], xv[MS][4];
    float s[NF], b[NF];
    auto fetch = [&](int c) {
        const int k0 = c * kChunk;
        const int g = (k0 + 32 * g4) / A.group;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            wv[f] = ld16g(wblk[f] + (size_t)c * 256);
            s[f] = bf16f(sblk[f][g * 16]);
            b[f] = bf16f(bblk[f][g * 16]);
        }
#pragma unroll
        for (int m = 0; m < MS; ++m)
#pragma unroll
            for (int st = 0; st < 4; ++st) xv[m][st] = ld16g(xrow[m] + k0 + 8 * st);
    };
    // each chunk's loads are issued while the one before computes (the last
    // chunk loads its own again: no branch around the loads)
    if (wave < nck) fetch(wave);
    for (int c = wave; c < nck; c += W) {
        uint4 wc[NF], xc[MS][4];
        float sc[NF], bc[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            wc[f] = wv[f];
            sc[f] = s[f];
            bc[f] = b[f];
        }
#pragma unroll
        for (int m = 0; m < MS; ++m)
#pragma unroll
            for (int st = 0; st < 4; ++st) xc[m][st] = xv[m][st];
        fetch(c + W < nck ? c + W : c);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const uint4 bw = dequant8(word(wc[f], st), sc[f], bc[f]);
#pragma unroll
                for (int m = 0; m < MS; ++m) acc[f][m] = mfma16x16x32(xc[m][st], bw, acc[f][m]);
            }
    }
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int m = 0; m < MS; ++m) red[wave][f * MS + m][lane] = acc[f][m];
    __syncthreads();
    // wave i < NF MS adds the partial sums of block i / MS, row tile i % MS
    // (waves in order)
    if (wave >= NF * MS) return;
    const int nb = blockIdx.x * NF + wave / MS, m = wave % MS;
    const int n = nb * 16 + l16;
    if (nb >= blocks || n >= features) return;
    f4v y = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) y += red[w][wave][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = r0 + 16 * m + 4 * g4 + i;
        if (r < A.rows) put(A, r, n, y[i]);
    }
}

// ---------------------------------------------------------------- decode
// The small kernel for 16 rows and at most 8 J chunks (J a wave): the same
// work, chunk order and sums, but every code word of a wave's J chunks is
// requested at the start, so that a workgroup holds all its weights in
// flight at once (80 KB at the 27B-like layer) instead of one chunk a wave;
// x (read from L2 by every workgroup) follows one chunk ahead, and the
// blocks' scales and biases come through LDS.  Loads retire in issue order:
// the first chunk waits only for its own codes, the later ones for all.
constexpr int kDecodeSbLoads = 3;   // 16-byte scale and bias loads a thread

template <int NF, int J>
__global__ void __launch_bounds__(512) inproj_decode_kernel(const InprojArgs A)
{
    constexpr int W = 8;
    __shared__ f4v red[W][NF][64];
    // the blocks' scales and biases, [f][group][16] bf16 each (groups of at
    // least 32 inputs: at most hidden / 32 of them, hidden <= 128 * 8 J)
    constexpr int kMaxGroups = 8 * J * kChunk / 32;
    __shared__ uint16_t ssb[2][NF][kMaxGroups * 16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int features = A.channels + 2 * A.hv;
    const int blocks = (features + 15) / 16;
    const int nck = A.hidden / kChunk, ng = A.hidden / A.group;
    // (past the last block, a workgroup's second block repeats the last one
    // and writes nothing)
    const uint32_t *wblk[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
        wblk[f] = A.wq + (size_t)min((int)blockIdx.x * NF + f, blocks - 1) * nck * 256 + 4 * lane;
    // scales and biases: at most kDecodeSbLoads 16-byte loads a thread (the
    // launch checks), requested first and parked in LDS, so that a wave's code and
    // x loads are not queued behind twenty 2-byte loads
    const int sbq = ng * 16 / 8;   // 16-byte pieces of one block's scales
    uint4 sbv[kDecodeSbLoads];
#pragma unroll
    for (int k2 = 0; k2 < kDecodeSbLoads; ++k2) {
        const int q = min(tid + 512 * k2, 2 * NF * sbq - 1);
        const int which = q / (NF * sbq), f = (q - which * NF * sbq) / sbq, e = q - (which * NF + f) * sbq;
        const int nb = min((int)blockIdx.x * NF + f, blocks - 1);
        sbv[k2] = ld16g((which ? A.biases : A.scales) + (size_t)nb * ng * 16 + 8 * e);
    }
    const uint16_t *xrow = A.x + (size_t)min(l16, A.rows - 1) * A.hidden + 32 * g4;
    // chunk j of this wave (past the end, the last chunk again: loaded, not used)
    auto chunk = [&](int j) { return min(wave + W * j, nck - 1); };
    uint4 xv[2][4];
    auto fetch_x = [&](int j, uint4 (&xd)[4]) {
#pragma unroll
        for (int st = 0; st < 4; ++st) xd[st] = ld16g(xrow + chunk(j) * kChunk + 8 * st);
    };
    fetch_x(0, xv[0]);
    uint4 wv[J][NF];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int f = 0; f < NF; ++f) wv[j][f] = ld16g(wblk[f] + (size_t)chunk(j) * 256);
#pragma unroll
    for (int k2 = 0; k2 < kDecodeSbLoads; ++k2) {
        const int q = tid + 512 * k2;
        if (q < 2 * NF * sbq) {
            const int which = q / (NF * sbq), f = (q - which * NF * sbq) / sbq, e = q - (which * NF + f) * sbq;
            *reinterpret_cast<uint4 *>(&ssb[which][f][8 * e]) = sbv[k2];
        }
    }
    lds_barrier();
    f4v acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < J; ++j) {
        if (j + 1 < J) fetch_x(j + 1, xv[(j + 1) & 1]);
        if (wave + W * j < nck) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const int g = (chunk(j) * kChunk + 32 * g4) / A.group;
                    acc[f] = mfma16x16x32(xv[j & 1][st],
                                          dequant8(word(wv[j][f], st), bf16f(ssb[0][f][g * 16 + l16]), bf16f(ssb[1][f][g * 16 + l16])),
                                          acc[f]);
                }
        }
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) red[wave][f][lane] = acc[f];
    __syncthreads();
    // wave f < NF adds the partial sums of block f (waves in order)
    if (wave >= NF) return;
    const int nb = blockIdx.x * NF + wave;
    const int n = nb * 16 + l16;
    if (nb >= blocks || n >= features) return;
    f4v y = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) y += red[w][wave][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        if (r < A.rows) put(A, r, n, y[i]);
    }
}

// ---------------------------------------------------------------- large
// A workgroup computes 64 WR rows x 128 features; wave (wr, wf) = (w >> 1,
// w & 1) the 64 x 64 block at rows 64 wr, features 64 wf, as 2 x 2
// v_mfma_f32_32x32x16_bf16 accumulators.  Inputs go in chunks of 64: the
// workgroup stages the chunk of x (64 WR x 64) and expands the chunk of
// weights (128 x 64: each thread 8 WPT inputs of one feature, WPT code words
// and one scale and bias) into LDS once, for all its waves; chunk c + 1's
// loads wait in registers and chunk c + 2's are in flight while chunk c
// computes (two LDS buffers).  WR = 4 (256 rows) halves the expansion work
// a product against WR = 2 and serves long launches.
// With KS = 2 (and WR = 2) a workgroup has two such groups of four waves,
// each with its own buffers and one half of the inputs; the second group's
// sums are added to the first's through LDS at the end (in that order).  Two
// groups a compute unit overlap one group's weight expansion and staging with
// the other's products: it serves launches with at most one tile a compute
// unit.
constexpr int kFeat = 128;             // features of a workgroup
constexpr int kKC = 64;                // inputs a chunk
constexpr int kPitch = kKC + 8;        // bf16 pitch of the staged rows (144 B)
constexpr int kYPitch = kFeat + 8;     // bf16 pitch of the output tile

template <int KS, int WR>
struct LargeCfg {
    static constexpr int rows = 64 * WR;                      // rows of a workgroup
    static constexpr int nt = 128 * WR;                       // threads of a share
    static constexpr int wpt = 8 / WR;                        // code words a thread a chunk
    static constexpr int xt = rows * kPitch;                  // staged x (bf16)
    static constexpr int buf = (rows + kFeat) * kPitch;       // one buffer: x and weights (bf16)
    static constexpr size_t lds = (size_t)KS * 2 * buf * sizeof(uint16_t);
};

__device__ __forceinline__ f16v mfma32x32x16(uint4 a, uint4 b, f16v c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8v, a), __builtin_bit_cast(bf8v, b), c,
                                                  0, 0, 0);
}

template <int KS, int WR>
__global__ void __launch_bounds__(128 * WR * KS) inproj_large_kernel(const InprojArgs A)
{
    using C = LargeCfg<KS, WR>;
    constexpr int NT = C::nt, WPT = C::wpt;
    extern __shared__ __align__(16) uint16_t lds_all[];   // [KS][2][x tile | weight tile]
    // kh: this thread's group (input share); tid, lane, wave within it
    const int kh = __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT);
    const int tid = threadIdx.x % NT, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint16_t *lds = lds_all + kh * 2 * C::buf;
    const int wr = wave >> 1, wf = wave & 1;
    const int l32 = lane & 31, hh = lane >> 5;
    const int features = A.channels + 2 * A.hv;
    const int ng = A.hidden / A.group, nck = A.hidden / kChunk;
    const int n0 = blockIdx.x * kFeat;
    const int r0 = blockIdx.y * C::rows;
    const int nchunks = A.hidden / kKC / KS;   // chunks of a share
    const int cbase = kh * nchunks;

    // this thread's staging: x pieces t + NT j (row p / 8, piece p % 8)
    const uint16_t *xsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int p = tid + NT * j;
        xsrc[j] = A.x + (size_t)min(r0 + (p >> 3), A.rows - 1) * A.hidden + 8 * (p & 7);
    }
    // weights: 128 / WPT threads a 16-feature block; thread t of a block
    // expands feature t % 16, inputs 8 WPT sub .. of a 64-input chunk (sub =
    // t / 16).  In the tiled layout those words sit in slot t % 16 + 16 g4 of
    // the chunk pair's 1 KB piece, g4 = 2 (c % 2) + input / 32, and the
    // threads of a block read 512 contiguous bytes.
    constexpr int TPB = 128 / WPT;
    const int bt = tid % TPB, l16 = bt & 15, sub = bt >> 4;
    const int f = 16 * (tid / TPB) + l16;
    const int ko = 8 * WPT * sub;   // first input within the chunk
    const int nb = min(n0 / 16 + tid / TPB, (features + 15) / 16 - 1);
    const uint32_t *wsrc = A.wq + (size_t)nb * nck * 256 + 4 * (l16 + 16 * (ko >> 5)) + ((ko & 31) >> 3);
    const uint16_t *ssrc = A.scales + (size_t)nb * ng * 16 + l16;
    const uint16_t *bsrc = A.biases + (size_t)nb * ng * 16 + l16;
    // a chunk's loads: its x pieces, this thread's code words, scale and bias
    // (kept as loaded: work on them here would wait for the loads)
    struct Loads {
        uint4 x[4];
        uint32_t w[WPT];
        uint32_t s, b;   // bf16 scale and bias
    };
    auto fetch = [&](int cs, Loads &L) {
        const int c = cbase + cs;
        const int k0 = c * kKC;
#pragma unroll
        for (int j = 0; j < 4; ++j) L.x[j] = ld16g(xsrc[j] + k0);
        // chunk pair c / 2, slots 32 (c % 2) ..
        const uint32_t *wc = wsrc + (size_t)(c >> 1) * 256 + 128 * (c & 1);
        if constexpr (WPT == 4) {
            const uint4 v = ld16g(wc);
            L.w[0] = v.x; L.w[1] = v.y; L.w[2] = v.z; L.w[3] = v.w;
        } else {
            const uint2 v = *reinterpret_cast<const uint2 *>(wc);
            L.w[0] = v.x; L.w[1] = v.y;
        }
        const int g = (k0 + ko) / A.group;
        L.s = ssrc[g * 16];
        L.b = bsrc[g * 16];
    };
    auto stage = [&](int bf, const Loads &L) {
        uint16_t *xt = lds + bf * C::buf, *wt = xt + C::xt;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = tid + NT * j;
            *reinterpret_cast<uint4 *>(xt + (p >> 3) * kPitch + 8 * (p & 7)) = L.x[j];
        }
        const float s = __uint_as_float(L.s << 16), b = __uint_as_float(L.b << 16);
#pragma unroll
        for (int i = 0; i < WPT; ++i)
            *reinterpret_cast<uint4 *>(wt + f * kPitch + ko + 8 * i) = dequant8(L.w[i], s, b);
    };

    f16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    // Step c computes chunk c from buffer c % 2 while chunk c + 2's loads
    // are in flight and chunk c + 1's wait in registers; these go to the
    // other buffer after the products, which every wave finished reading
    // before the barrier that ended step c - 1.  The two register sets trade
    // roles from step to step (a copy from one to the other would wait for
    // the loads in flight).  Past the end, the last chunk is loaded again:
    // no branch around the loads.
    Loads la, lb;
    fetch(0, la);
    stage(0, la);
    fetch(min(1, nchunks - 1), la);
    lds_barrier();
    auto step = [&](int c, const Loads &cur, Loads &nxt) {
        fetch(min(c + 2, nchunks - 1), nxt);
        const uint16_t *xt = lds + (c & 1) * C::buf, *wt = xt + C::xt;
        const uint16_t *xa = xt + (64 * wr + l32) * kPitch + 8 * hh;
        const uint16_t *wb = wt + (64 * wf + l32) * kPitch + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < kKC / 16; ++ks) {
            const uint4 a0 = *reinterpret_cast<const uint4 *>(xa + 16 * ks);
            const uint4 a1 = *reinterpret_cast<const uint4 *>(xa + 32 * kPitch + 16 * ks);
            const uint4 b0 = *reinterpret_cast<const uint4 *>(wb + 16 * ks);
            const uint4 b1 = *reinterpret_cast<const uint4 *>(wb + 32 * kPitch + 16 * ks);
            acc[0][0] = mfma32x32x16(a0, b0, acc[0][0]);
            acc[0][1] = mfma32x32x16(a0, b1, acc[0][1]);
            acc[1][0] = mfma32x32x16(a1, b0, acc[1][0]);
            acc[1][1] = mfma32x32x16(a1, b1, acc[1][1]);
        }
        stage((c + 1) & 1, cur);
        lds_barrier();
    };
    int c = 0;
    for (; c + 1 < nchunks; c += 2) {
        step(c, la, lb);
        step(c + 1, lb, la);
    }
    if (c < nchunks) step(c, la, lb);

    if constexpr (KS == 2) {
        // the second share's sums, [wave][i][j][e][lane] in fp32, through the
        // second share's buffers (every wave is past the barrier after its
        // last chunk)
        static_assert(64 * 4 * 64 * sizeof(float) * (WR / 2) <= 2 * C::buf * sizeof(uint16_t), "partials");
        float *part = reinterpret_cast<float *>(lds_all + 2 * C::buf);
        if (kh == 1) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) part[(((wave * 2 + i) * 2 + j) * 16 + e) * 64 + lane] = acc[i][j][e];
        }
        lds_barrier();
        if (kh == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] += part[(((wave * 2 + i) * 2 + j) * 16 + e) * 64 + lane];
        }
    }

    // accumulator register e of lane (l32, hh) of block (i, j): row
    // 64 wr + 32 i + 8 (e / 4) + 4 hh + e % 4, feature 64 wf + 32 j + l32;
    // the first share writes the tile
    if (n0 + kFeat <= A.channels) {
        // inside qkv: the tile through LDS (the first share's two buffers;
        // every wave is past the barrier after the last chunk), then 16-byte
        // stores of whole 256-byte row pieces
        static_assert(C::rows * kYPitch <= 2 * C::buf, "output tile");
        uint16_t *ys = lds_all;
        if (kh == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        ys[(64 * wr + 32 * i + 8 * (e >> 2) + 4 * hh + (e & 3)) * kYPitch + 64 * wf + 32 * j + l32] =
                            f2bf(acc[i][j][e]);
        }
        lds_barrier();
        if (kh != 0) return;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int p = tid + NT * j;   // row p / 16, piece p % 16
            const int r = r0 + (p >> 4);
            if (r < A.rows)
                *reinterpret_cast<uint4 *>(A.qkv + (size_t)r * A.channels + n0 + 8 * (p & 15)) =
                    *reinterpret_cast<const uint4 *>(ys + (p >> 4) * kYPitch + 8 * (p & 15));
        }
        return;
    }
    if (kh != 0) return;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = n0 + 64 * wf + 32 * j + l32;
        if (n >= features) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = r0 + 64 * wr + 32 * i + 8 * (e >> 2) + 4 * hh + (e & 3);
                if (r < A.rows) put(A, r, n, acc[i][j][e]);
            }
    }
}

// ---------------------------------------------------------------- repack
// MLX layout -> tiled layout, one thread a word quad (and, for the first
// K / group threads of a block row, its scales and biases).
__global__ void __launch_bounds__(256) inproj_pack_kernel(const InprojPackArgs P)
{
    const int features = P.channels + 2 * P.hv;
    const int nck = P.hidden / kChunk, kw = P.hidden / 8, ng = P.hidden / P.group;
    const size_t quads = (size_t)P.blocks * nck * 64;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < quads) {
        const int lane = (int)(i & 63);
        const size_t bc = i >> 6;                      // block * nck + chunk
        const int nb = (int)(bc / nck), c = (int)(bc - (size_t)nb * nck);
        const int n = nb * 16 + (lane & 15), g4 = lane >> 4;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (n < features) {
            const uint32_t *src = P.wq + (size_t)n * kw + 16 * c + 4 * g4;
            v = make_uint4(src[0], src[1], src[2], src[3]);
        }
        *reinterpret_cast<uint4 *>(P.wq_tiled + 4 * i) = v;
    }
    const size_t sbn = (size_t)P.blocks * ng * 16;
    if (i < sbn) {
        const int l16 = (int)(i & 15);
        const size_t bg = i >> 4;                      // block * ng + group
        const int nb = (int)(bg / ng), g = (int)(bg - (size_t)nb * ng);
        const int n = nb * 16 + l16;
        P.scales_tiled[i] = n < features ? P.scales[(size_t)n * ng + g] : (uint16_t)0;
        P.biases_tiled[i] = n < features ? P.biases[(size_t)n * ng + g] : (uint16_t)0;
    }
}

// Compute units of the current device (looked up once per device; a race
// between threads writes the same value).
int compute_units()
{
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

template <int KS, int WR>
hipError_t launch_large(const InprojArgs &A, int ft, hipStream_t stream)
{
    using C = LargeCfg<KS, WR>;
    static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(inproj_large_kernel<KS, WR>),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((inproj_large_kernel<KS, WR>), dim3(ft, (A.rows + C::rows - 1) / C::rows), dim3(C::nt * KS),
                       C::lds, stream, A);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_inproj_pack(const InprojPackArgs &P, hipStream_t stream)
{
    const size_t quads = (size_t)P.blocks * (P.hidden / kChunk) * 64;
    const size_t sbn = (size_t)P.blocks * (P.hidden / P.group) * 16;
    const size_t n = quads > sbn ? quads : sbn;
    hipLaunchKernelGGL(inproj_pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, P);
    return hipGetLastError();
}

hipError_t launch_inproj(const InprojArgs &A, hipStream_t stream)
{
    const int features = A.channels + 2 * A.hv;
    if (A.rows <= 32) {
        const int blocks = (features + 15) / 16;
        // up to 16 rows and 40 chunks (hidden 5120): every weight requested
        // up front.  Each workgroup reads all of x, so it takes as many
        // feature blocks (up to 3) as leave workgroups for three quarters of
        // the compute units (the 27B-like layer: 3, 216 workgroups), while
        // the blocks' scales and biases fit the kernel's loads
        const int J = (A.hidden / kChunk + 7) / 8;
        int nfd = 1;
        for (int c = 3; c >= 2; --c)
            if (4 * ((blocks + c - 1) / c) >= 3 * compute_units()) {
                nfd = c;
                break;
            }
        if (A.rows <= 16 && J <= 5 && 4 * nfd * (A.hidden / A.group) <= 512 * kDecodeSbLoads) {
            const dim3 grid((blocks + nfd - 1) / nfd, 1);
            switch (nfd * 8 + J) {
#define GDN_DECODE(NF, J) \
    case NF * 8 + J: hipLaunchKernelGGL((inproj_decode_kernel<NF, J>), grid, dim3(512), 0, stream, A); break;
                GDN_DECODE(1, 1) GDN_DECODE(1, 2) GDN_DECODE(1, 3) GDN_DECODE(1, 4) GDN_DECODE(1, 5)
                GDN_DECODE(2, 1) GDN_DECODE(2, 2) GDN_DECODE(2, 3) GDN_DECODE(2, 4) GDN_DECODE(2, 5)
                GDN_DECODE(3, 1) GDN_DECODE(3, 2) GDN_DECODE(3, 3) GDN_DECODE(3, 4) GDN_DECODE(3, 5)
#undef GDN_DECODE
            }
            return hipGetLastError();
        }
        // otherwise two feature blocks a workgroup while that still leaves a
        // workgroup for every compute unit
        const int nf = blocks / 2 >= compute_units() ? 2 : 1;
        const dim3 grid((blocks + nf - 1) / nf, A.rows <= 16 ? (A.rows + 15) / 16 : (A.rows + 31) / 32);
        if (A.rows <= 16) {
            if (nf == 2) hipLaunchKernelGGL((inproj_small_kernel<1, 2>), grid, dim3(512), 0, stream, A);
            else hipLaunchKernelGGL((inproj_small_kernel<1, 1>), grid, dim3(512), 0, stream, A);
        } else {
            if (nf == 2) hipLaunchKernelGGL((inproj_small_kernel<2, 2>), grid, dim3(512), 0, stream, A);
            else hipLaunchKernelGGL((inproj_small_kernel<2, 1>), grid, dim3(512), 0, stream, A);
        }
    } else {
        // two input shares a workgroup while 128-row tiles leave a compute
        // unit to each workgroup; 256-row tiles for long launches
        const int ft = (features + kFeat - 1) / kFeat;
        const int t128 = ft * ((A.rows + 127) / 128);
        if (t128 <= compute_units()) return launch_large<2, 2>(A, ft, stream);
        if (A.rows > 512) return launch_large<1, 4>(A, ft, stream);
        return launch_large<1, 2>(A, ft, stream);
    }
    return hipGetLastError();
}

}  // namespace gdn
