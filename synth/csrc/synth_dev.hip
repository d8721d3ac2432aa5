// Seeded synthetic inputs for the Stable LatentMoE layer: device twin.
//
// Bit-for-bit the same values as the host twin in synth_host.c (same
// counter-based SplitMix64 words, same 65536-entry normal-quantile table, same
// fp32 multiply and bf16 / e2m1 rounding); it exists only so that tens of GB of
// synthetic weights can be written straight into HBM. It holds none of the
// layer's arithmetic. The table is passed in as a device pointer.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t GOLD = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t word_at(uint64_t key, uint64_t c) {
  return mix64(key + (c + 1) * GOLD);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float mul_rn(float a, float b) { return __fmul_rn(a, b); }

// Each thread makes the four elements that share one 64-bit word.
template <typename OutT>
__global__ void normal_kernel(uint64_t key, uint64_t start, int64_t n, float sigma,
                              const float* __restrict__ table, OutT* __restrict__ out) {
  const int64_t w0 = (int64_t)(start >> 2);
  const int64_t w1 = (int64_t)((start + (uint64_t)n + 3) >> 2);
  for (int64_t w = w0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < w1;
       w += (int64_t)gridDim.x * blockDim.x) {
    uint64_t bits = word_at(key, (uint64_t)w);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      int64_t i = w * 4 + h - (int64_t)start;
      if (i < 0 || i >= n) continue;
      float v = mul_rn(table[(bits >> (16 * h)) & 0xFFFFu], sigma);
      if constexpr (sizeof(OutT) == 2) out[i] = bf16_rne(v);
      else out[i] = v;
    }
  }
}

__device__ __forceinline__ uint32_t e2m1_code(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

// One thread per 32-element block along K.
__global__ void mxfp4_kernel(uint64_t key, uint64_t row0, int64_t rows, int64_t K, float sigma,
                             const float* __restrict__ table, uint8_t* __restrict__ packed,
                             uint8_t* __restrict__ scales) {
  const int64_t nblk = K / 32;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < rows * nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = b / nblk, kb = b % nblk;
    uint64_t base = (row0 + (uint64_t)r) * (uint64_t)K + (uint64_t)(kb * 32);
    uint16_t m[32];
    uint32_t amax = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint64_t bits = word_at(key, (base >> 2) + q);   // base is a multiple of 32
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint16_t v = bf16_rne(mul_rn(table[(bits >> (16 * h)) & 0xFFFFu], sigma));
        m[q * 4 + h] = v;
        uint32_t a = v & 0x7FFFu;
        amax = a > amax ? a : amax;
      }
    }
    uint8_t* dst = packed + r * (K / 2) + kb * 16;
    if (amax == 0) {
      scales[r * nblk + kb] = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[i] = 0;
      continue;
    }
    int e;
    uint32_t ef = (amax >> 7) & 0xFFu;
    if (ef != 0) {
      e = (int)ef - 127;
    } else {
      uint32_t mant = amax & 0x7Fu;
      int p = 6;
      while (!(mant & (1u << p))) --p;
      e = -133 + p;
    }
    int x = e - 2;
    x = x < -127 ? -127 : (x > 127 ? 127 : x);
    scales[r * nblk + kb] = (uint8_t)(x + 127);
    double inv = ldexp(1.0, -x);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint8_t byte = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v = __uint_as_float((uint32_t)m[2 * i + h] << 16);
        float q = (float)((double)v * inv);
        uint32_t code = e2m1_code(fabsf(q));
        if (q < 0.0f || (v == 0.0f && signbit(v))) code |= 8u;
        byte |= (uint8_t)(code << (4 * h));
      }
      dst[i] = byte;
    }
  }
}

int grid_for(int64_t work) {
  int64_t g = (work + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

int synth_dev_normal_f32(uint64_t key, uint64_t start, int64_t n, float sigma,
                         const float* table, float* out, void* stream) {
  if (n <= 0) return 0;
  int64_t words = (int64_t)(((start + (uint64_t)n + 3) >> 2) - (start >> 2));
  hipLaunchKernelGGL(normal_kernel<float>, dim3(grid_for(words)), dim3(256), 0,
                     (hipStream_t)stream, key, start, n, sigma, table, out);
  return (int)hipGetLastError();
}

int synth_dev_normal_bf16(uint64_t key, uint64_t start, int64_t n, float sigma,
                          const float* table, uint16_t* out, void* stream) {
  if (n <= 0) return 0;
  int64_t words = (int64_t)(((start + (uint64_t)n + 3) >> 2) - (start >> 2));
  hipLaunchKernelGGL(normal_kernel<uint16_t>, dim3(grid_for(words)), dim3(256), 0,
                     (hipStream_t)stream, key, start, n, sigma, table, out);
  return (int)hipGetLastError();
}

int synth_dev_mxfp4(uint64_t key, uint64_t row0, int64_t rows, int64_t K, float sigma,
                    const float* table, uint8_t* packed, uint8_t* scales, void* stream) {
  if (rows <= 0) return 0;
  if (K % 32 != 0) return 1;
  hipLaunchKernelGGL(mxfp4_kernel, dim3(grid_for(rows * (K / 32))), dim3(256), 0,
                     (hipStream_t)stream, key, row0, rows, K, sigma, table, packed, scales);
  return (int)hipGetLastError();
}

}  // extern "C"
