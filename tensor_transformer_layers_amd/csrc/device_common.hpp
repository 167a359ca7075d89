// device_common.hpp -- vector types and small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte global load / store (the natural width of one lane's MFMA operand chunk).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v)
{
    return bf16x4{to_bf16(v[0]), to_bf16(v[1]), to_bf16(v[2]), to_bf16(v[3])};
}

__device__ __forceinline__ f32x4 bf16x4_to_f32(bf16x4 v)
{
    return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
                 static_cast<float>(v[3])};
}

// Phi(x), the standard normal CDF, as erfc(-x / sqrt 2) / 2. erfc(z) for z >= 0 comes from
// the Chebyshev fit of Numerical Recipes (Press, Teukolsky, Vetterling and Flannery, 2nd ed.,
// section 6.2, function erfcc): erfc(z) = t exp(-z^2 + P(t)) with t = 1 / (1 + z / 2) and a
// degree-9 polynomial P, fractional error below 1.2e-7 for every z >= 0. For x < 0 this gives
// Phi(x) = erfc(|x| / sqrt 2) / 2 to that relative accuracy all the way into the tail (no
// 1 + erf(x) cancellation); for x >= 0, 1 - erfc / 2. Branch-free: one reciprocal, nine
// FMAs, one exp, where a general-purpose erff branches on the argument's range and divergent
// lanes pay for every range.
__device__ __forceinline__ float normal_cdf(float x)
{
    const float z = fabsf(x) * 0.70710678118654752440f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
    float q = fmaf(t, 0.17087277f, -0.82215223f);
    q = fmaf(t, q, 1.48851587f);
    q = fmaf(t, q, -1.13520398f);
    q = fmaf(t, q, 0.27886807f);
    q = fmaf(t, q, -0.18628806f);
    q = fmaf(t, q, 0.09678418f);
    q = fmaf(t, q, 0.37409196f);
    q = fmaf(t, q, 1.00002368f);
    q = fmaf(t, q, -1.26551223f);
    const float half_erfc = 0.5f * t * __expf(q - z * z);
    return x >= 0.0f ? 1.0f - half_erfc : half_erfc;
}

// Exact GeLU, x * Phi(x), in fp32.
__device__ __forceinline__ float gelu_erf(float x)
{
    return x * normal_cdf(x);
}

// Derivative of the exact GeLU: Phi(x) + x phi(x), phi the standard normal density.
__device__ __forceinline__ float gelu_erf_grad(float x)
{
    return normal_cdf(x) + x * 0.39894228040143267794f * __expf(-0.5f * x * x);
}

// D = A * B + C on a 16x16 output block with K = 32 (bf16 in, fp32 accumulate).
// Lane l supplies A row (l & 15) and B column (l & 15), 8 consecutive K values each, and
// receives D rows 4 * (l >> 4) + i, i = 0..3, of column (l & 15).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A * B + C on a 32x32 output block with K = 16 (bf16 in, fp32 accumulate).
// Lane l supplies A row (l & 31) and B column (l & 31), 8 consecutive K values each, and
// receives D rows 8 * j + 4 * (l >> 5) + i (accumulator element 4 j + i) of column (l & 31).
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Same block shape with fp32 operands and K = 4: lane l supplies one K value, (l >> 4).
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace tps
