// Quantile Balancing: the per-expert selection bias from quantiles of the
// router scores.
//
// "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか" (lilting.ch),
// section "ルーター専用の独立訓練はない": for each expert, the boundary score at
// which it would receive its target number of tokens is read off as a
// quantile of its score distribution, and the selection bias is updated from
// it (during training; inference keeps the final bias fixed). "Kimi K3
// テクニカルレポート" (jiwasawa.github.io), section "幅のスケーリング: Stable
// LatentMoE": the quantiles come directly from histograms of the router
// scores, with no auxiliary loss.
//
// Here, for a batch of T tokens and target c = round(T k / E) tokens per
// expert: q_e = the c-th largest score s[t][e] over t (exact), tau = the mean
// of q over the experts (fp64 sum, e ascending, rounded to fp32), and
// b_e = fp32(tau - q_e): after the update each expert has exactly c tokens
// whose score sits at or above its boundary q_e = tau - b_e, and the common
// shift tau leaves every top-k choice unchanged. The c-th largest value is
// found by radix selection: four passes of 256-bin histograms over the 8-bit
// digits of the order-preserving integer code of the score, each pass keeping
// the keys that match the digits chosen so far (integer counts: the result
// does not depend on the order of the additions).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// Order-preserving map of an fp32 value to uint32 (larger value -> larger
// code; -0 and +0 share one code) and its inverse.
__device__ __forceinline__ uint32_t qb_code(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float qb_decode(uint32_t c) {
  return __uint_as_float((c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c);
}

constexpr int kQbExperts = 4;    // experts per block (enough blocks to spread over the CUs)
constexpr int kQbGroups = 64;    // token groups per block (256 threads)

// Block: experts e0 .. e0 + 3; thread (g, l) reads expert e0 + l of tokens
// t = g (mod 64), so 4 neighbouring lanes read one 16-byte piece of a token's
// scores (the blocks of neighbouring experts share the rest of the line in L2).
__global__ __launch_bounds__(256) void qb_select_kernel(const float* __restrict__ s, int T, int E,
                                                        int c, float* __restrict__ q) {
  __shared__ uint32_t hist[kQbExperts][256];
  __shared__ uint32_t prefix[kQbExperts], need[kQbExperts];
  const int l = threadIdx.x % kQbExperts, g = threadIdx.x / kQbExperts;
  const int e = blockIdx.x * kQbExperts + l;
  if (threadIdx.x < kQbExperts) {
    prefix[threadIdx.x] = 0;
    need[threadIdx.x] = (uint32_t)c;
  }
  uint32_t mask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < kQbExperts * 256; i += blockDim.x) (&hist[0][0])[i] = 0;
    __syncthreads();
    if (e < E) {
      const uint32_t pre = prefix[l];
      for (int t = g; t < T; t += kQbGroups) {
        const uint32_t key = qb_code(s[(int64_t)t * E + e]);
        if ((key & mask) == pre) atomicAdd(&hist[l][(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (threadIdx.x < kQbExperts && e < E) {
      // the digit of the c-th largest key: walk the bins from the top
      uint32_t cum = 0, r = need[l];
      for (int dgt = 255; dgt >= 0; --dgt) {
        const uint32_t h = hist[l][dgt];
        if (cum + h >= r) {
          prefix[l] |= (uint32_t)dgt << shift;
          need[l] = r - cum;
          break;
        }
        cum += h;
      }
    }
    mask |= 255u << shift;
    __syncthreads();
  }
  if (threadIdx.x < kQbExperts && e < E) q[e] = qb_decode(prefix[l]);
}

// tau = fp32(sum_e q_e / E), the sum in fp64 with e ascending (one thread);
// b_e = fp32(tau - q_e).
__global__ __launch_bounds__(256) void qb_bias_kernel(const float* __restrict__ q, int E,
                                                      float* __restrict__ b) {
  __shared__ float tau;
  if (threadIdx.x == 0) {
    double sum = 0.0;
    for (int e = 0; e < E; ++e) sum += (double)q[e];
    tau = (float)(sum / (double)E);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) b[e] = __fsub_rn(tau, q[e]);
}

}  // namespace

int qb_target(int T, int E, int k) {
  const int64_t c = ((int64_t)T * k + E / 2) / E;   // round(T k / E), ties up
  return (int)(c < 1 ? 1 : (c > T ? T : c));
}

int launch_qb_bias(const float* scores, int T, int E, int k, float* q, float* bias,
                   hipStream_t stream) {
  if (T == 0) return -1;
  hipLaunchKernelGGL(qb_select_kernel, dim3((unsigned)ceil_div(E, kQbExperts)), dim3(256), 0, stream,
                     scores, T, E, qb_target(T, E, k), q);
  hipLaunchKernelGGL(qb_bias_kernel, dim3(1), dim3(256), 0, stream, q, E, bias);
  return (int)hipGetLastError();
}

}  // namespace moe
