// Affine 4-bit in-projection of libgdn (gfx950): the mixer's inputs qkv, a
// and b from hidden rows x, y = x W^T, with W stored as 4-bit codes and a
// bf16 scale and bias per output feature and group of inputs
// (w = s * q + b; page "perf(qwen3_5 cuda): deliver the first token before
// drafting", the note on the MLX affine 4-bit checkpoint, whose projections
// run through affine-4 kernels; the format is MLX's affine quantisation).
//
// Each weight is expanded to bf16 (s * q + b in fp32, rounded to nearest
// even) right before it enters v_mfma_f32_16x16x32_bf16, as MLX's own matrix
// kernels do; products accumulate in fp32 and the outputs are rounded to bf16.
//
// Inputs go in chunks of 128.  Within a chunk, lane (l16, g4) of a wave owns
// inputs [32 g4, 32 g4 + 32): four consecutive code words, one 16-byte load,
// and in k-step s (0..3) it supplies inputs 32 g4 + 8 s .. + 8 of both
// operands (A: row l16 of x, B: feature l16 of W), so that every input meets
// its weight once.  Its 32 inputs lie in one group (group sizes 32, 64, 128),
// so one scale and one bias serve the lane for the chunk.
//
//   small  (rows <= 32): a workgroup is 16 features x 16 or 32 rows; its four
//          waves take every fourth chunk and add their partial sums in LDS.
//   large  a workgroup is 64 features x 128 rows, wave w the features
//          [16 w, 16 w + 16) of all 128 rows (8 accumulators); the chunk of x
//          is staged in LDS for the four waves, and the output tile leaves
//          through LDS in whole 128-byte rows where it lies inside qkv.
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
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fmaf(s, (float)((w >> (4 * j)) & 15u), b);
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
template <int MS>
__global__ void __launch_bounds__(256) inproj_small_kernel(const InprojArgs A)
{
    __shared__ f4v red[4][MS][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int features = A.channels + 2 * A.hv;
    const int kw = A.hidden / 8, ng = A.hidden / A.group;
    const int n = blockIdx.x * 16 + l16;
    const int nl = min(n, features - 1);
    const int r0 = blockIdx.y * 16 * MS;
    const uint32_t *wrow = A.wq + (size_t)nl * kw + 4 * g4;
    const uint16_t *xrow[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) xrow[m] = A.x + (size_t)min(r0 + 16 * m + l16, A.rows - 1) * A.hidden + 32 * g4;

    f4v acc[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) acc[m] = f4v{0.f, 0.f, 0.f, 0.f};
    for (int c = wave; c < A.hidden / kChunk; c += 4) {
        const int k0 = c * kChunk;
        const uint4 wv = ld16g(wrow + k0 / 8);
        const int g = (k0 + 32 * g4) / A.group;
        const float s = bf16f(A.scales[(size_t)nl * ng + g]);
        const float b = bf16f(A.biases[(size_t)nl * ng + g]);
        uint4 xv[MS][4];
#pragma unroll
        for (int m = 0; m < MS; ++m)
#pragma unroll
            for (int st = 0; st < 4; ++st) xv[m][st] = ld16g(xrow[m] + k0 + 8 * st);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint4 bw = dequant8(word(wv, st), s, b);
#pragma unroll
            for (int m = 0; m < MS; ++m) acc[m] = mfma16x16x32(xv[m][st], bw, acc[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < MS; ++m) red[wave][m][lane] = acc[m];
    __syncthreads();
    if (wave != 0 || n >= features) return;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        const f4v y = ((red[0][m][lane] + red[1][m][lane]) + red[2][m][lane]) + red[3][m][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + 16 * m + 4 * g4 + i;
            if (r < A.rows) put(A, r, n, y[i]);
        }
    }
}

// ---------------------------------------------------------------- large
constexpr int kRows = 128;             // rows of a workgroup
constexpr int kXPitch = kChunk + 8;    // bf16 pitch of the staged x rows (272 B: rows 4 banks apart)
constexpr int kYPitch = 64 + 8;        // bf16 pitch of the output tile

__global__ void __launch_bounds__(256) inproj_large_kernel(const InprojArgs A)
{
    __shared__ __align__(16) uint16_t xs[kRows * kXPitch];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int features = A.channels + 2 * A.hv;
    const int kw = A.hidden / 8, ng = A.hidden / A.group;
    const int n0 = blockIdx.x * 64;
    const int n = n0 + 16 * wave + l16;
    const int nl = min(n, features - 1);
    const int r0 = blockIdx.y * kRows;
    const uint32_t *wrow = A.wq + (size_t)nl * kw + 4 * g4;

    // staging: thread t moves 16-byte pieces t + 256 j (row p / 16, piece p % 16)
    const uint16_t *xsrc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int p = tid + 256 * j;
        xsrc[j] = A.x + (size_t)min(r0 + (p >> 4), A.rows - 1) * A.hidden + 8 * (p & 15);
    }

    f4v acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = f4v{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < A.hidden / kChunk; ++c) {
        const int k0 = c * kChunk;
        uint4 xv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = ld16g(xsrc[j] + k0);
        const uint4 wv = ld16g(wrow + k0 / 8);
        const int g = (k0 + 32 * g4) / A.group;
        const float s = bf16f(A.scales[(size_t)nl * ng + g]);
        const float b = bf16f(A.biases[(size_t)nl * ng + g]);
        lds_barrier();   // every wave is done with the previous chunk
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int p = tid + 256 * j;
            *reinterpret_cast<uint4 *>(xs + (p >> 4) * kXPitch + 8 * (p & 15)) = xv[j];
        }
        lds_barrier();
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint4 bw = dequant8(word(wv, st), s, b);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint4 av = *reinterpret_cast<const uint4 *>(xs + (16 * m + l16) * kXPitch + 32 * g4 + 8 * st);
                acc[m] = mfma16x16x32(av, bw, acc[m]);
            }
        }
    }

    if (n0 + 64 <= A.channels) {
        // inside qkv: the tile [128 rows][64 features] through LDS, then rows
        // of 128 bytes (16-byte stores)
        lds_barrier();
        uint16_t *ys = xs;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) ys[(16 * m + 4 * g4 + i) * kYPitch + 16 * wave + l16] = f2bf(acc[m][i]);
        lds_barrier();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = tid + 256 * j;   // row p / 8, piece p % 8
            const int r = r0 + (p >> 3);
            if (r < A.rows)
                *reinterpret_cast<uint4 *>(A.qkv + (size_t)r * A.channels + n0 + 8 * (p & 7)) =
                    *reinterpret_cast<const uint4 *>(ys + (p >> 3) * kYPitch + 8 * (p & 7));
        }
        return;
    }
    if (n >= features) return;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + 16 * m + 4 * g4 + i;
            if (r < A.rows) put(A, r, n, acc[m][i]);
        }
}

}  // namespace

hipError_t launch_inproj(const InprojArgs &A, hipStream_t stream)
{
    const int features = A.channels + 2 * A.hv;
    if (A.rows <= 16) {
        hipLaunchKernelGGL(inproj_small_kernel<1>, dim3((features + 15) / 16, (A.rows + 15) / 16), dim3(256), 0,
                           stream, A);
    } else if (A.rows <= 32) {
        hipLaunchKernelGGL(inproj_small_kernel<2>, dim3((features + 15) / 16, (A.rows + 31) / 32), dim3(256), 0,
                           stream, A);
    } else {
        hipLaunchKernelGGL(inproj_large_kernel, dim3((features + 63) / 64, (A.rows + kRows - 1) / kRows), dim3(256),
                           0, stream, A);
    }
    return hipGetLastError();
}

}  // namespace gdn
