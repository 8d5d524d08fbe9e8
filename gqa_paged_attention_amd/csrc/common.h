// Internal helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// log2(e): scores are carried in base-2 units so that one v_exp_f32 gives e^x.
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_inff();
// A running maximum is only raised when a block's maximum exceeds it by more
// than this many base-2 units, so unnormalised weights stay below 2^8 and the
// accumulators are rescaled rarely.  The final division uses the same
// reference point, so the result does not depend on it.
constexpr float kRescaleSlack = 8.0f;

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, each as 8 consecutive-k values of
// lane group l / 16; it receives D rows 4 * (l / 16) + i, i = 0..3, of column
// l % 16.  A and B share one k order, so only row/column placement matters.
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 values to packed bf16 (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// The low (sel = 0) or high (sel = 1) 16-bit halves of a and b, a's in bits 0..15.
__device__ __forceinline__ uint32_t pair_half(uint32_t a, uint32_t b, int sel)
{
    return sel ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Reduce over the four lanes l, l^16, l^32, l^48 (the four lane groups that
// hold one MFMA column).
__device__ __forceinline__ float group4_max(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

__device__ __forceinline__ float group4_sum(float v)
{
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}

}  // namespace attn
