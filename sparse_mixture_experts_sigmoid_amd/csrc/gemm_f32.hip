// fp32 kernels of the Stable LatentMoE layer (activations and weights fp32).
//
// Same equations as the bf16 matrix-core path (see gemm.hip): z = W_down x,
// the routed experts' gated FFN with SiTU-GLU on permuted rows, and the output
// GEMM whose K runs over the shared experts' down projections and W_up. These
// serve the small all-fp32 layer, a parity case rather than a throughput
// target, so each output element is one thread's fp32 fma chain.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ float dot_f32(const float* a, const float* b, int K) {
  float acc = 0.0f;
  for (int k = 0; k < K; ++k) acc = __builtin_fmaf(a[k], b[k], acc);
  return acc;
}

__global__ void dense_f32(DenseArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.M * a.N) return;
  const int m = (int)(i / a.N), n = (int)(i % a.N);
  ((float*)a.C)[(int64_t)m * a.ldc + n] =
      dot_f32((const float*)a.A + (int64_t)m * a.lda, (const float*)a.W.data + (int64_t)n * a.K, a.K);
}

__global__ void glu_f32(GluArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.M * a.F) return;
  const int m = (int)(i / a.F), f = (int)(i % a.F);
  const float* x = (const float*)a.A + (int64_t)m * a.lda;
  float g = dot_f32(x, (const float*)a.Wg.data + (int64_t)f * a.K, a.K);
  float v = dot_f32(x, (const float*)a.Wv.data + (int64_t)f * a.K, a.K);
  ((float*)a.H)[(int64_t)m * a.ldh + f] = situ_glu(g, v, a.c, 1.0f / a.c);
}

__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E;  // offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void grouped_glu_f32(GroupedGluArgs a) {
  const int64_t rows = min((int64_t)a.offsets[a.E], (int64_t)a.rows_cap);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * a.F) return;
  const int r = (int)(i / a.F), f = (int)(i % a.F);
  const int e = expert_of_row(a.offsets, a.E, r);
  const int src = a.perm_src[r];
  if (src < 0 || src / a.topk >= a.T) return;
  const float* z = (const float*)a.Z + (int64_t)(src / a.topk) * a.ldz;
  const int64_t wrow = (int64_t)e * a.F + f;
  float g = dot_f32(z, (const float*)a.Wg.data + wrow * a.K, a.K);
  float v = dot_f32(z, (const float*)a.Wv.data + wrow * a.K, a.K);
  ((float*)a.H)[(int64_t)r * a.F + f] = situ_glu(g, v, a.c, 1.0f / a.c);
}

__global__ void grouped_down_f32(GroupedDownArgs a) {
  const int64_t rows = min((int64_t)a.offsets[a.E], (int64_t)a.rows_cap);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * a.N) return;
  const int r = (int)(i / a.N), n = (int)(i % a.N);
  const int e = expert_of_row(a.offsets, a.E, r);
  ((float*)a.O)[(int64_t)r * a.N + n] =
      dot_f32((const float*)a.H + (int64_t)r * a.ldh,
              (const float*)a.Wo.data + ((int64_t)e * a.N + n) * a.K, a.K);
}

__global__ void multiseg_f32(MultiSegArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.M * a.N) return;
  const int m = (int)(i / a.N), n = (int)(i % a.N);
  float acc = 0.0f;
  for (int s = 0; s < a.nseg; ++s) {
    const Segment& sg = a.seg[s];
    const float* x = (const float*)sg.A + (int64_t)m * sg.lda;
    const float* w = (const float*)sg.B.data + (int64_t)n * sg.K;
    for (int k = 0; k < sg.K; ++k) acc = __builtin_fmaf(x[k], w[k], acc);
  }
  ((float*)a.C)[(int64_t)m * a.ldc + n] = acc;
}

unsigned blocks_for(int64_t n) { return (unsigned)ceil_div(n, 256); }

}  // namespace

int launch_dense_f32(const DenseArgs& a, hipStream_t stream) {
  if (a.M == 0) return 0;
  hipLaunchKernelGGL(dense_f32, dim3(blocks_for((int64_t)a.M * a.N)), dim3(256), 0, stream, a);
  return (int)hipGetLastError();
}

int launch_glu_f32(const GluArgs& a, hipStream_t stream) {
  if (a.M == 0) return 0;
  hipLaunchKernelGGL(glu_f32, dim3(blocks_for((int64_t)a.M * a.F)), dim3(256), 0, stream, a);
  return (int)hipGetLastError();
}

// rows <= max_tiles: the fp32 path uses one-row tiles
int launch_grouped_glu_f32(const GroupedGluArgs& a, hipStream_t stream) {
  if (a.max_tiles == 0) return 0;
  hipLaunchKernelGGL(grouped_glu_f32, dim3(blocks_for((int64_t)a.max_tiles * a.F)), dim3(256), 0,
                     stream, a);
  return (int)hipGetLastError();
}

int launch_grouped_down_f32(const GroupedDownArgs& a, hipStream_t stream) {
  if (a.max_tiles == 0) return 0;
  hipLaunchKernelGGL(grouped_down_f32, dim3(blocks_for((int64_t)a.max_tiles * a.N)), dim3(256), 0,
                     stream, a);
  return (int)hipGetLastError();
}

int launch_multiseg_f32(const MultiSegArgs& a, hipStream_t stream) {
  if (a.M == 0) return 0;
  hipLaunchKernelGGL(multiseg_f32, dim3(blocks_for((int64_t)a.M * a.N)), dim3(256), 0, stream, a);
  return (int)hipGetLastError();
}

}  // namespace moe
