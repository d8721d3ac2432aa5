// Weighted combine + RMSNorm.
//
// "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか" (lilting.ch,
// section "K3のエキスパートは896個の小型LLMではない"): u = sum_{i in Top16} p_i E_i(z),
// then RMSNorm(u) feeds W_up. Token-centric gather (no atomics, so the sum
// order is fixed: slots in order j = 0..k-1): one block per token reads its k
// expert rows through inv_pos, accumulates in fp32, reduces sum(u^2) across
// the block and writes n = u / sqrt(mean(u^2) + eps) * gain.
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

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  extern __shared__ float u_s[];
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int64_t rows = (int64_t)a.T * a.k;
  const T* O = (const T*)a.O;
  const float* g = a.gate + (int64_t)t * a.k;
  const int32_t* ip = a.inv_pos + (int64_t)t * a.k;

  float ss = 0.0f;
  for (int i = threadIdx.x; i < a.D; i += blockDim.x) {
    float u = 0.0f;
    for (int j = 0; j < a.k; ++j) {
      const int64_t r = ip[j];
      if (r < 0 || r >= rows) continue;
      u = __builtin_fmaf(g[j], load_f32(O, r * a.D + i), u);
    }
    u_s[i] = u;
    ss = __builtin_fmaf(u, u, ss);
  }
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)a.D + a.eps);
  T* n = (T*)a.n_out + (int64_t)t * a.ldn;
  for (int i = threadIdx.x; i < a.D; i += blockDim.x) {
    const float u = u_s[i];
    if (a.u_out) a.u_out[(int64_t)t * a.D + i] = u;
    store_f32(n, i, u * inv * (a.gain ? a.gain[i] : 1.0f));
  }
}

}  // namespace

int launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T == 0) return 0;
  const size_t lds = (size_t)a.D * sizeof(float);
  if (a.act_dtype == DT_F32)
    hipLaunchKernelGGL(combine_kernel<float>, dim3(a.T), dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(a.T), dim3(256), lds, stream, a);
  return (int)hipGetLastError();
}

}  // namespace moe
