// MXFP8 quantisation of activation rows for the scaled-MFMA expert GEMMs.
//
// OCP Microscaling (MX) v1.0, E4M3 elements: per block of 32 consecutive
// elements along K, X = floor(log2 amax) - 8 (8 is the largest E4M3
// exponent; clamped to [-127, 127], amax = 0 gives -127), stored as the e8m0
// byte X + 127; element code = the E4M3 value nearest to v / 2^X (ties to
// even), saturating at +-448, sign bit set when v < 0. Every step is exact
// except the one rounding (v / 2^X is a power-of-two scaling of a bf16 value;
// the mantissa rounding is rintf in the default round-to-nearest-even mode).
// MXFP4 weights ("Kimi K3 ... Open Frontier Intelligence", section "MXFP4
// Quantization-Aware Training") meet these activations in the gfx950 scaled
// MFMA, which takes both operands in MX formats.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// floor(log2 |y|) of a normal fp32 value from its exponent field
__device__ __forceinline__ int exp_field(float y) { return (int)((__float_as_uint(y) >> 23) & 0xFFu) - 127; }

// E4M3 code of y = |v| / 2^X (0 <= y < 512)
__device__ __forceinline__ uint32_t e4m3_mag(float y) {
  if (y < 0x1p-6f) return (uint32_t)__builtin_rintf(y * 512.0f);   // subnormal steps of 2^-9 (8 -> 0x08)
  int e = exp_field(y);
  uint32_t m = (uint32_t)__builtin_rintf((__builtin_ldexpf(y, -e) - 1.0f) * 8.0f);
  if (m == 8u) { m = 0u; ++e; }
  const uint32_t code = ((uint32_t)(e + 7) << 3) | m;
  return (y >= 448.0f || code > 0x7Eu) ? 0x7Eu : code;
}

// One thread per 8 consecutive elements (a 16-byte bf16 load); the 4 threads
// of a 32-element block are adjacent lanes and share amax through shuffles.
__global__ __launch_bounds__(256) void quantize_mx8_kernel(const bf16_t* __restrict__ in, int64_t rows,
                                                           int K, int64_t ld, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const int per_row = K / 8;
  const int64_t n = rows * per_row;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g - (threadIdx.x & 63) < n;
       g += (int64_t)gridDim.x * blockDim.x) {
    // every lane of the wave runs the shuffles (a wave is 8 whole blocks: 64 % 4 == 0,
    // per_row % 4 == 0); lanes past the end work on zeros and store nothing
    const bool live = g < n;
    const int64_t row = live ? g / per_row : 0;
    const int c8 = live ? (int)(g % per_row) : 0;
    uint4 v = live ? *(const uint4*)(in + row * ld + (int64_t)c8 * 8) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    // X = floor(log2 amax) - 8; a zero or subnormal amax has exponent field 0 -> -127
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
    const int X = ef == 0 ? -127 : max(-127, min(127, ef - 127 - 8));
    uint32_t q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = __builtin_ldexpf(fabsf(x[i]), -X);
      q[i] = e4m3_mag(y) | (x[i] < 0.0f ? 0x80u : 0u);
    }
    if (live) {
      const uint32_t lo = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
      const uint32_t hi = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
      *(uint2*)(codes + row * K + (int64_t)c8 * 8) = make_uint2(lo, hi);
      if ((c8 & 3) == 0) scales[row * (K / 32) + c8 / 4] = (uint8_t)(X + 127);
    }
  }
}

}  // namespace

int launch_quantize_mx8(const void* in, int64_t rows, int K, int64_t ld, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream) {
  if (rows == 0) return 0;
  if (K % 32) return -1;
  const int64_t n = rows * (K / 8);
  const int64_t blocks = ceil_div(n, 256) < 8192 ? ceil_div(n, 256) : 8192;
  hipLaunchKernelGGL(quantize_mx8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const bf16_t*)in, rows, K, ld, codes, scales);
  return (int)hipGetLastError();
}

}  // namespace moe
