// Shared device helpers of the gfx950 Stable LatentMoE kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage dtypes (same values as moe_dtype_t).
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_MXFP4 = 2 };

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void store_f32(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_f32<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_f32<bf16_t>(bf16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// SiTU-GLU in fp32: c*tanh(SiLU(g)/c) * c*tanh(v/c). e^x through the hardware
// 2^x; tanh(a) = 1 - 2/(e^{2a}+1) away from 0 (saturates cleanly at both
// ends) and its odd Taylor polynomial to a^7 for |a| < 1/8 (no cancellation).
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504f); }

__device__ __forceinline__ float tanh_fast(float a) {
  if (fabsf(a) < 0.125f) {
    float a2 = a * a;
    return a * (1.0f + a2 * (-0.333333333f + a2 * (0.133333333f + a2 * -0.0539682540f)));
  }
  float e = exp_fast(2.0f * a);
  return 1.0f - __fdividef(2.0f, e + 1.0f);
}

__device__ __forceinline__ float situ_glu(float g, float v, float c, float inv_c) {
  float silu = __fdividef(g, 1.0f + exp_fast(-g));
  return (c * tanh_fast(silu * inv_c)) * (c * tanh_fast(v * inv_c));
}

// Buffer resources: loads at offsets past num_records return zeros (no fault).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;  // past every buffer (each is < 2^31 bytes)

// Every resource is built from block-uniform values; readfirstlane states that
// to the compiler so the descriptor lives in scalar registers (a descriptor in
// vector registers turns each load into a waterfall loop).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n,
                                           0x00020000);
}

__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
