// MXFP8 quantisation of activation rows for the scaled-MFMA expert GEMMs.
//
// OCP Microscaling (MX) v1.0, E4M3 elements: per block of 32 consecutive
// elements along K, X = floor(log2 amax) - 8 (8 is the largest E4M3
// exponent; clamped to [-127, 127], amax = 0 gives -127), stored as the e8m0
// byte X + 127; element code = the E4M3 value nearest to v / 2^X (ties to
// even), saturating at +-448, sign bit set when v < 0. Every step is exact
// except the one rounding (v / 2^X is a power-of-two scaling of a bf16 value),
// which gfx950's v_cvt_pk_fp8_f32 performs.
// MXFP4 weights ("Kimi K3 ... Open Frontier Intelligence", section "MXFP4
// Quantization-Aware Training") meet these activations in the gfx950 scaled
// MFMA, which takes both operands in MX formats.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// A thread converts runs of 8 consecutive elements (a 16-byte bf16 load); the 4
// threads of a 32-element block are adjacent lanes and share amax through
// shuffles.
constexpr int kU = 8;

__device__ __forceinline__ void quantize_run(const uint4 v, bool live, int64_t row, int c8, int K,
                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
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
  // gfx950's v_cvt_pk_fp8_f32 rounds to the nearest OCP E4M3 value (ties to
  // even, subnormals kept) and keeps the sign; clamping to +-448 first gives the
  // saturation. The input gets + 0.0f, which turns -0.0 into +0.0 (no sign bit
  // for v = 0) and leaves every other value as it is, so a negative v whose
  // scaled value underflows to -0.0 still gets the sign bit
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(__builtin_ldexpf(x[i] + 0.0f, -X), -448.0f), 448.0f);
  uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)lo, true);
  uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)hi, true);
  if (live) {
    *(uint2*)(codes + row * K + (int64_t)c8 * 8) = make_uint2(lo, hi);
    if ((c8 & 3) == 0) scales[row * (K / 32) + c8 / 4] = (uint8_t)(X + 127);
  }
}

// One wave per row at a time: lane l takes the 8-element runs l, l + 64, ...
// of the row, all kU of a pass loaded before any is converted. No division on
// the index path; a wave's lanes past the row's end work on zeros and store
// nothing (a 4-lane group is wholly live or wholly idle, as K % 32 == 0).
__global__ __launch_bounds__(256) void quantize_mx8_kernel(const bf16_t* __restrict__ in, int64_t rows,
                                                           int K, int64_t ld, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const int per_row = K / 8;
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); row < rows; row += waves) {
    const bf16_t* src = in + row * ld;
    for (int c0 = 0; c0 < per_row; c0 += 64 * kU) {
      uint4 v[kU];
      bool live[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c8 = c0 + 64 * u + lane;
        live[u] = c8 < per_row;
        v[u] = live[u] ? *(const uint4*)(src + (int64_t)c8 * 8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) quantize_run(v[u], live[u], row, c0 + 64 * u + lane, K, codes, scales);
    }
  }
}

// One thread per output dword: the 4 scale bytes (one 128-element stage) of
// one row, read as a dword from the row-major array (K/32 % 4 == 0 keeps it
// aligned) and written where the tiled layout puts them, so that consecutive
// threads write consecutive dwords.
__global__ __launch_bounds__(256) void tile_scales_kernel(const uint32_t* __restrict__ in,
                                                          uint32_t* __restrict__ out, int64_t rows,
                                                          int nk) {
  const int64_t n = rows * nk;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tile = i / (64 * (int64_t)nk);
    const int rem = (int)(i - tile * 64 * nk);
    const int kt = rem >> 6, rl = rem & 63;
    out[i] = in[(tile * 64 + rl) * nk + kt];
  }
}

// One thread per output 16-byte chunk of the packed bytes: chunk c (0..3) of
// row 2p + h's stage kt, with h = which row of the pair.
__global__ __launch_bounds__(256) void pair_rows_kernel(const uint4* __restrict__ in, uint4* __restrict__ out,
                                                        int64_t rows, int nk) {
  const int64_t n = rows * nk * 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t pair = i / (8 * (int64_t)nk);
    const int rem = (int)(i - pair * 8 * nk);
    const int kt = rem >> 3, h = (rem >> 2) & 1, c = rem & 3;
    out[i] = in[(2 * pair + h) * (4 * (int64_t)nk) + 4 * kt + c];
  }
}

}  // namespace

int launch_tile_mxfp4(const uint8_t* data, const uint8_t* scale, uint8_t* data_out, uint8_t* scale_out,
                      int64_t rows, int K, hipStream_t stream) {
  if (rows % 64 || K % 128 || ((uintptr_t)scale | (uintptr_t)scale_out) % 4 ||
      ((uintptr_t)data | (uintptr_t)data_out) % 16)
    return -1;
  if (rows == 0) return 0;
  const int nk = K / 128;
  const int64_t nd = rows * nk * 4, ns = rows * nk;
  hipLaunchKernelGGL(pair_rows_kernel, dim3((unsigned)(ceil_div(nd, 256) < 16384 ? ceil_div(nd, 256) : 16384)),
                     dim3(256), 0, stream, (const uint4*)data, (uint4*)data_out, rows, nk);
  hipLaunchKernelGGL(tile_scales_kernel, dim3((unsigned)(ceil_div(ns, 256) < 16384 ? ceil_div(ns, 256) : 16384)),
                     dim3(256), 0, stream, (const uint32_t*)scale, (uint32_t*)scale_out, rows, nk);
  return (int)hipGetLastError();
}

int launch_quantize_mx8(const void* in, int64_t rows, int K, int64_t ld, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream) {
  if (rows == 0) return 0;
  if (K % 32) return -1;
  const int64_t blocks = ceil_div(rows, 4) < 8192 ? ceil_div(rows, 4) : 8192;
  hipLaunchKernelGGL(quantize_mx8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const bf16_t*)in, rows, K, ld, codes, scales);
  return (int)hipGetLastError();
}

}  // namespace moe
