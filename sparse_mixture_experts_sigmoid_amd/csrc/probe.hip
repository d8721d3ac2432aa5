// Ceiling probes of one MI355X, the measured denominators that bench.py
// reports beside the published peaks: back-to-back matrix-core instructions
// with no memory traffic (bf16 and MXFP8 x MXFP4, each with fixed or with
// changing operands), and a plain streaming read of HBM. Not part of the layer: libmoe_probe.so is loaded by bench.py only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

// As mfma_bf16_kernel, but with operands that change at every instruction:
// four A and four B fragments of pseudo-random bf16 values in [-2, 2) (from a
// hash of the lane), each chain stepping through the 16 pairs, so that the
// matrix cores switch on data like a real GEMM (their power, and with it the
// clock, depends on it).
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}
__global__ __launch_bounds__(256) void mfma_bf16_data_kernel(int iters, float* out) {
  bf16x8 a[4], b[4];
  for (int u = 0; u < 4; ++u)
    for (int i = 0; i < 8; ++i) {
      const uint32_t ha = probe_hash(threadIdx.x * 64u + u * 8u + i + 1u);
      const uint32_t hb = probe_hash(threadIdx.x * 64u + u * 8u + i + 0x9e3779b9u);
      a[u][i] = (__bf16)((float)(ha & 0xFFFFu) * (4.0f / 65536.0f) - 2.0f);
      b[u][i] = (__bf16)((float)(hb & 0xFFFFu) * (4.0f / 65536.0f) - 2.0f);
    }
  f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(u + c) & 3], b[(u + 2 * c + (c >> 1)) & 3], acc[c], 0, 0, 0);
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// NT: nontemporal loads (streamed past the caches' normal retention).
// BLK: each block reads one contiguous part of the buffer (gridDim parts, in
// spans of U x 256 chunks) from its start to its end, as a GEMM block streams
// its own weight slice; otherwise the spans are handed out grid-stride.
template <int U, bool NT, bool BLK>
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                       uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const int64_t span = (int64_t)U * 256;
  const int64_t part = (n16 + (int64_t)gridDim.x * span - 1) / ((int64_t)gridDim.x * span) * span;
  const int64_t b0 = BLK ? (int64_t)blockIdx.x * part : (int64_t)blockIdx.x * span;
  const int64_t b1 = BLK ? (b0 + part < n16 ? b0 + part : n16) : n16;
  const int64_t step = BLK ? span : (int64_t)gridDim.x * span;
  for (int64_t b = b0; b < b1; b += step) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = b + u * 256 + threadIdx.x;
      if (i < b1) v[u] = NT ? __builtin_nontemporal_load(p + i) : p[i];
      else v[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// As mfma_f8f4_kernel, but with pseudo-random E4M3 and E2M1 codes that change
// at every instruction (four A and four B operand sets per lane, as above).
// E4M3 codes 0x7f / 0xff (NaN) are mapped to 0x7e / 0xfe.
__global__ __launch_bounds__(256) void mfma_f8f4_data_kernel(int iters, float* out) {
  v8i a[4], b[4];
  for (int u = 0; u < 4; ++u)
    for (int i = 0; i < 8; ++i) {
      uint32_t ha = probe_hash(threadIdx.x * 64u + u * 8u + i + 7u);
      const uint32_t hb = probe_hash(threadIdx.x * 64u + u * 8u + i + 0x85ebca6bu);
      for (int k = 0; k < 4; ++k) {        // no NaN bytes
        const uint32_t byte = (ha >> (8 * k)) & 0xFFu;
        if ((byte & 0x7Fu) == 0x7Fu) ha ^= 1u << (8 * k);
      }
      a[u][i] = (int)ha;
      b[u][i] = i < 4 ? (int)hb : 0;
    }
  f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(u + c) & 3], b[(u + 2 * c + (c >> 1)) & 3],
                                                                 acc[c], 0, 4, 0, 127, 0, 127);
  }
  float s = 0.0f;
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = s;
}

// v_mfma_f32_16x16x32_bf16 (the same FLOP rate per clock as 32x32x16 on paper,
// half the FLOP per instruction), 8 independent accumulators per wave: fixed
// operands (DATA = false) or the changing ones of mfma_bf16_data_kernel.
template <bool DATA>
__global__ __launch_bounds__(256) void mfma_bf16_16_kernel(int iters, float* out) {
  bf16x8 a[4], b[4];
  for (int u = 0; u < 4; ++u)
    for (int i = 0; i < 8; ++i) {
      const uint32_t ha = probe_hash(threadIdx.x * 64u + u * 8u + i + 1u);
      const uint32_t hb = probe_hash(threadIdx.x * 64u + u * 8u + i + 0x9e3779b9u);
      a[u][i] = DATA ? (__bf16)((float)(ha & 0xFFFFu) * (4.0f / 65536.0f) - 2.0f) : (__bf16)(float)((threadIdx.x + i) & 7);
      b[u][i] = DATA ? (__bf16)((float)(hb & 0xFFFFu) * (4.0f / 65536.0f) - 2.0f) : (__bf16)(float)((threadIdx.x * 3 + i) & 7);
    }
  f32x4 acc[2 * kChains];
  for (int c = 0; c < 2 * kChains; ++c)
    for (int r = 0; r < 4; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 2 * kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(u + c) & 3], b[(u + 2 * c + (c >> 1)) & 3], acc[c], 0, 0, 0);
  }
  float s = 0.0f;
  for (int c = 0; c < 2 * kChains; ++c)
    for (int r = 0; r < 4; ++r) s += acc[c][r];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = s;
}

}  // namespace

extern "C" {

int moe_probe_mfma(int kind, int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr || kind < 0 || kind > 5 || (kind >= 2 && iters % 4)) return -1;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_f8f4_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  else if (kind == 2)
    hipLaunchKernelGGL(mfma_bf16_data_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  else if (kind == 3)
    hipLaunchKernelGGL(mfma_f8f4_data_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  else if (kind == 4)
    hipLaunchKernelGGL(mfma_bf16_16_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  else
    hipLaunchKernelGGL(mfma_bf16_16_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

double moe_probe_mfma_flops(int kind, int blocks, int iters) {
  if (kind >= 4) return 2.0 * 16 * 16 * 32 * (2 * kChains) * 4.0 * blocks * (double)iters;
  const double per = (kind == 1 || kind == 3) ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
  return per * kChains * 4.0 * blocks * (double)iters;   // 4 waves per block
}

int moe_probe_hbm_read(const void* buf, int64_t bytes, int blocks, int unroll, uint32_t* out, void* stream) {
  const int u = unroll & 0xFF;
  const bool nt = (unroll & 0x100) != 0, blk = (unroll & 0x200) != 0;
  if (buf == nullptr || out == nullptr || bytes <= 0 || bytes % 16 || blocks <= 0 ||
      ((uintptr_t)buf & 15u) || (u != 4 && u != 8 && u != 16) || (unroll & ~0x3FF))
    return -1;
  const u32x4* p = (const u32x4*)buf;
  hipStream_t s = (hipStream_t)stream;
  const int64_t n = bytes / 16;
#define MOE_HBM_READ(U, NT, BLK) \
  hipLaunchKernelGGL((hbm_read_kernel<U, NT, BLK>), dim3(blocks), dim3(256), 0, s, p, n, out)
#define MOE_HBM_READ_U(NT, BLK)         \
  do {                                  \
    if (u == 4) MOE_HBM_READ(4, NT, BLK);   \
    else if (u == 8) MOE_HBM_READ(8, NT, BLK); \
    else MOE_HBM_READ(16, NT, BLK);        \
  } while (0)
  if (!nt && !blk) MOE_HBM_READ_U(false, false);
  else if (nt && !blk) MOE_HBM_READ_U(true, false);
  else if (!nt) MOE_HBM_READ_U(false, true);
  else MOE_HBM_READ_U(true, true);
#undef MOE_HBM_READ_U
#undef MOE_HBM_READ
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
