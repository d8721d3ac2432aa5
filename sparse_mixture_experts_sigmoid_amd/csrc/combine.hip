// Weighted combine + RMSNorm.
//
// "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか" (lilting.ch,
// section "K3のエキスパートは896個の小型LLMではない"): u = sum_{i in Top16} p_i E_i(z),
// then RMSNorm(u) feeds W_up. Token-centric gather (no atomics, so the sum
// order is fixed: slots in order j = 0..k-1, one fp32 fma each): one block per
// token reads its k expert rows through inv_pos, reduces sum(u^2) across the
// block and writes n = u / sqrt(mean(u^2) + eps) * gain.
//
// bf16 rows: each thread owns CPT chunks of 8 consecutive elements (one
// 16-byte load per row and chunk), keeps u in registers, and issues the loads
// of up to 8 rows before their fmas, so a thread has that many row reads in
// flight. fp32 rows (the small all-fp32 layer): one element per thread step.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float s = 0.0f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}

__device__ __forceinline__ void fma8(float (&u)[8], float g, uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u[2 * i] = __builtin_fmaf(g, __uint_as_float(w[i] << 16), u[2 * i]);
    u[2 * i + 1] = __builtin_fmaf(g, __uint_as_float(w[i] & 0xFFFF0000u), u[2 * i + 1]);
  }
}

constexpr int kRowBatch = 8;   // rows whose loads are in flight together

template <int CPT>
__global__ __launch_bounds__(1024) void combine_bf16_kernel(CombineArgs a) {
  __shared__ float red[16];
  const int t = blockIdx.x;
  const int64_t rows = (int64_t)a.T * a.k;
  const int nch = a.D / 8;
  const bf16_t* O = (const bf16_t*)a.O;
  const float* g = a.gate + (int64_t)t * a.k;
  const int32_t* ip = a.inv_pos + (int64_t)t * a.k;

  float u[CPT][8];
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) u[c][i] = 0.0f;

  for (int j0 = 0; j0 < a.k; j0 += kRowBatch) {
    uint4 v[kRowBatch][CPT];
#pragma unroll
    for (int jj = 0; jj < kRowBatch; ++jj) {
      const int j = j0 + jj;
      const int64_t r = j < a.k ? ip[j] : -1;
      const bool ok = r >= 0 && r < rows;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int ch = threadIdx.x + c * blockDim.x;
        v[jj][c] = (ok && ch < nch) ? *(const uint4*)(O + r * a.D + ch * 8) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int jj = 0; jj < kRowBatch; ++jj) {
      if (j0 + jj >= a.k) break;
      const float gj = g[j0 + jj];
      // a row that is not there (inv_pos < 0) read zeros: gj * 0 adds nothing
#pragma unroll
      for (int c = 0; c < CPT; ++c) fma8(u[c], gj, v[jj][c]);
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(u[c][i], u[c][i], ss);
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)a.D + a.eps);
  bf16_t* n = (bf16_t*)a.n_out + (int64_t)t * a.ldn;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * blockDim.x;
    if (ch >= nch) continue;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = ch * 8 + 2 * i;
      const float g0 = a.gain ? a.gain[e] : 1.0f, g1 = a.gain ? a.gain[e + 1] : 1.0f;
      w[i] = (uint32_t)f32_to_bf16(u[c][2 * i] * inv * g0) |
             ((uint32_t)f32_to_bf16(u[c][2 * i + 1] * inv * g1) << 16);
    }
    *(uint4*)(n + ch * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    if (a.u_out) {
      float* uo = a.u_out + (int64_t)t * a.D + ch * 8;
      *(float4*)uo = make_float4(u[c][0], u[c][1], u[c][2], u[c][3]);
      *(float4*)(uo + 4) = make_float4(u[c][4], u[c][5], u[c][6], u[c][7]);
    }
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(CombineArgs a) {
  extern __shared__ float u_s[];
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int64_t rows = (int64_t)a.T * a.k;
  const float* O = (const float*)a.O;
  const float* g = a.gate + (int64_t)t * a.k;
  const int32_t* ip = a.inv_pos + (int64_t)t * a.k;

  float ss = 0.0f;
  for (int i = threadIdx.x; i < a.D; i += blockDim.x) {
    float u = 0.0f;
    for (int j = 0; j < a.k; ++j) {
      const int64_t r = ip[j];
      if (r < 0 || r >= rows) continue;
      u = __builtin_fmaf(g[j], O[r * a.D + i], u);
    }
    u_s[i] = u;
    ss = __builtin_fmaf(u, u, ss);
  }
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)a.D + a.eps);
  float* n = (float*)a.n_out + (int64_t)t * a.ldn;
  for (int i = threadIdx.x; i < a.D; i += blockDim.x) {
    const float u = u_s[i];
    if (a.u_out) a.u_out[(int64_t)t * a.D + i] = u;
    n[i] = u * inv * (a.gain ? a.gain[i] : 1.0f);
  }
}

}  // namespace

int launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T == 0) return 0;
  if (a.act_dtype == DT_F32) {
    hipLaunchKernelGGL(combine_f32_kernel, dim3(a.T), dim3(256), (size_t)a.D * sizeof(float), stream, a);
    return (int)hipGetLastError();
  }
  // bf16: D % 8 == 0 (the layer's dims are multiples of 32); chunks of 8 per thread
  const int nch = a.D / 8;
  const int cpt = (int)ceil_div(nch, 1024);
  const int threads = (int)ceil_div(ceil_div(nch, cpt), 64) * 64;
  if (cpt == 1) hipLaunchKernelGGL(combine_bf16_kernel<1>, dim3(a.T), dim3(threads), 0, stream, a);
  else if (cpt == 2) hipLaunchKernelGGL(combine_bf16_kernel<2>, dim3(a.T), dim3(threads), 0, stream, a);
  else if (cpt <= 4) hipLaunchKernelGGL(combine_bf16_kernel<4>, dim3(a.T), dim3(threads), 0, stream, a);
  else return -1;
  return (int)hipGetLastError();
}

}  // namespace moe
