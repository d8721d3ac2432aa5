// Ceiling probes of one MI355X, the measured denominators that bench.py
// reports beside the published peaks: back-to-back matrix-core instructions
// with no memory traffic (bf16 and MXFP8 x MXFP4), and a plain streaming read
// of HBM. Not part of the layer: libmoe_probe.so is loaded by bench.py only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kChains = 4;   // independent accumulators per wave (waves per SIMD give the rest)

// Each wave: `iters` rounds of kChains independent v_mfma_f32_32x32x16_bf16.
// The operands come from the thread index (never constant-folded); one lane
// per wave writes a sum of its accumulators so nothing is dead code.
__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, float* out) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
    b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 7);
  }
  f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = s;
}

// Same with v_mfma_scale_f32_32x32x64_f8f6f4, A in E4M3 and B in E2M1
// (format selectors 0 and 4), unit scales (e8m0 byte 127).
__global__ __launch_bounds__(256) void mfma_f8f4_kernel(int iters, float* out) {
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)(0x38383838u + ((threadIdx.x + i) & 3));
    b[i] = i < 4 ? (int)(0x22222222u + ((threadIdx.x + i) & 1)) : 0;
  }
  f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 4, 0, 127, 0, 127);
  }
  float s = 0.0f;
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = s;
}

// Each block reads contiguous spans of U x 256 16-byte chunks (all U loads of
// a thread issued before any is used), spans handed out grid-stride; each
// thread folds what it read into one word that it writes, so every load is live.
template <int U>
__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                       uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const int64_t span = (int64_t)U * 256;
  for (int64_t b = (int64_t)blockIdx.x * span; b < n16; b += (int64_t)gridDim.x * span) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = b + u * 256 + threadIdx.x;
      v[u] = i < n16 ? p[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

int moe_probe_mfma(int kind, int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr || (kind != 0 && kind != 1)) return -1;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  else
    hipLaunchKernelGGL(mfma_f8f4_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

double moe_probe_mfma_flops(int kind, int blocks, int iters) {
  const double per = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  return per * kChains * 4.0 * blocks * (double)iters;   // 4 waves per block
}

int moe_probe_hbm_read(const void* buf, int64_t bytes, int blocks, int unroll, uint32_t* out, void* stream) {
  if (buf == nullptr || out == nullptr || bytes <= 0 || bytes % 16 || blocks <= 0 ||
      ((uintptr_t)buf & 15u) || (unroll != 4 && unroll != 8 && unroll != 16))
    return -1;
  const uint4* p = (const uint4*)buf;
  hipStream_t s = (hipStream_t)stream;
  if (unroll == 4) hipLaunchKernelGGL(hbm_read_kernel<4>, dim3(blocks), dim3(256), 0, s, p, bytes / 16, out);
  else if (unroll == 8) hipLaunchKernelGGL(hbm_read_kernel<8>, dim3(blocks), dim3(256), 0, s, p, bytes / 16, out);
  else hipLaunchKernelGGL(hbm_read_kernel<16>, dim3(blocks), dim3(256), 0, s, p, bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
