// Device helpers shared by libgdn's kernel files (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16f(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }

typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even: gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two fp32 values -> packed bf16 bits (lo in bits 0..15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    const bf2v v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// The gates, SiLU and the norms use the hardware's exp2, log2, reciprocal and
// reciprocal square root (about 1 ulp each; the IEEE sequences are 5 to 40
// times as many instructions, 131 for log1pf(expf(x))), every kernel the same
// functions, so window rows and one-row steps still agree bit for bit.

// softplus(x) = log(1 + e^x) without overflow.  For x < -17 the log term
// rounds to 0 (the true value is below e^-17 of the result's unit, and the
// decay it feeds differs from 1 by less than an fp32 ulp).
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.0f) + __logf(1.0f + __expf(-fabsf(x))); }

__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// log of the per-row decay: g = -exp(A_log) softplus(a + dt_bias), alpha = e^g.
__device__ __forceinline__ float log_decay(float a, float a_log, float dt_bias)
{
    return -__expf(a_log) * softplus_f(a + dt_bias);
}

// the decay alpha = e^g
__device__ __forceinline__ float decay_f(float g) { return __expf(g); }

// SiLU of a conv output: y * sigmoid(y)
__device__ __forceinline__ float silu_f(float y) { return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y)); }

// 1 / sqrt(sum of squares + eps) of an L2 norm
__device__ __forceinline__ float inv_norm_f(float ss) { return __builtin_amdgcn_rsqf(ss + 1e-6f); }

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

// Sum over each 16-lane row of the wave with DPP lane moves (no LDS round
// trip); every lane of the row gets the same bits, the bits of the xor
// butterfly over masks 1, 2, 4, 8.  quad_perm [1,0,3,2] and [2,3,0,1] sum each
// quad, row_half_mirror the two quads of each half-row (every lane of a quad
// holds the quad's sum), row_mirror the two half-rows.
__device__ __forceinline__ float sum_row16(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}

// Sum over the eight 8-lane groups of the wave (lanes l, l^8, ..., l^56);
// every lane gets the same bits.  row_ror:8 pairs each lane with lane ^ 8
// inside its 16-lane row, then permlane16_swap and permlane32_swap as above.
__device__ __forceinline__ float sum_rows8(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    return sum_rows4(x);
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

// Wait until every vector memory operation of the wave has completed
// (s_waitcnt vmcnt(0), expcnt and lgkmcnt left alone).  A real waitcnt
// instruction, which the compiler's own wait insertion takes into account.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load and store of the thread (its fence covers
// global memory), which would hold each barrier on loads and stores in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace gdn
