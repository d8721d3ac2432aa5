// Router (s = Sigmoid(W_r x), key = s + b) and wavefront top-k + gates.
//
// Source: "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか"
// (lilting.ch), section "ルーターは計算の割当器": the router projects the hidden
// state to one sigmoid score per expert, adds a per-expert balancing bias to
// choose the top-k, and normalises the chosen experts' unbiased scores into the
// mixing weights.
//
// The top-k choice is discrete, so the scores are computed by one fixed fp32
// sequence that a CPU can repeat bit for bit: per (token, expert) the chain
// acc = fma(x_k, w_k, acc) over k ascending from +0 (no split-K, no MFMA: the
// matrix cores do not expose their internal summation order), then the sigmoid
// below, built only from correctly rounded IEEE-754 operations.
//
// This file is compiled with -ffp-contract=off: every fma is written out.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// Constants of the fixed sigmoid, each the fp32 rounding of its exact value:
// ln2 split as LN2_HI + LN2_LO (LN2_HI = fp32(ln 2), LN2_LO = fp32(ln 2 - LN2_HI)),
// log2(e), and 1/j! for j = 0..7.
constexpr float kLn2Hi = 0x1.62e430p-1f;
constexpr float kLn2Lo = -0x1.05c610p-29f;
constexpr float kLog2e = 0x1.715476p+0f;
constexpr float kInvFact[8] = {0x1.0p+0f,     0x1.0p+0f,     0x1.0p-1f,     0x1.555556p-3f,
                               0x1.555556p-5f, 0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f};

// sigmoid(l) = 1 / (1 + e^a), a = -l clamped to [-87, 87]:
// n = rint(a * log2 e) (ties to even); r = a - n ln2 in two fma steps (Cody &
// Waite); e^r by the degree-7 Taylor polynomial in Horner form with fma; e^a =
// 2^n e^r by exact scaling; then one correctly rounded division.
__device__ __forceinline__ float sigmoid_fixed(float l) {
  float a = -l;
  a = a > 87.0f ? 87.0f : a;
  a = a < -87.0f ? -87.0f : a;
  float n = __builtin_rintf(__fmul_rn(a, kLog2e));
  float r = __builtin_fmaf(-n, kLn2Hi, a);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = kInvFact[7];
#pragma unroll
  for (int j = 6; j >= 0; --j) p = __builtin_fmaf(p, r, kInvFact[j]);
  float e = __builtin_ldexpf(p, (int)n);
  return __fdiv_rn(1.0f, __fadd_rn(1.0f, e));
}

// Router GEMM on the vector ALUs. Block = 16 x 16 threads; thread (ty, tx)
// owns a TM x TN micro-tile: tokens t0 + ty*TM + i, experts e0 + tx*TN + j.
// x and W_r are staged through LDS in K-chunks of KC, k-major (transposed) so a
// thread reads its TM (TN) consecutive values with one vector load.
template <int TM, int TN, typename XT, typename WT>
__global__ __launch_bounds__(256) void router_kernel(const XT* __restrict__ x,
                                                     const WT* __restrict__ W,
                                                     const float* __restrict__ bias, int T,
                                                     int d, int E, float* __restrict__ s_out,
                                                     float* __restrict__ key_out) {
  constexpr int BT = 16 * TM, BE = 16 * TN, KC = 32;
  __shared__ float xs[KC][BT + 4];
  __shared__ float ws[KC][BE + 4];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int t0 = blockIdx.y * BT, e0 = blockIdx.x * BE;

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

  for (int kc = 0; kc < d; kc += KC) {
    const int kn = min(KC, d - kc);
    // cooperative loads (zero-fill outside the matrix; those lanes are never used
    // by an FMA because the inner loop stops at kn and rows outside are discarded)
    for (int idx = threadIdx.x; idx < BT * KC; idx += 256) {
      int r = idx / KC, kk = idx % KC;
      int t = t0 + r;
      xs[kk][r] = (t < T && kk < kn) ? load_f32(x, (int64_t)t * d + kc + kk) : 0.0f;
    }
    for (int idx = threadIdx.x; idx < BE * KC; idx += 256) {
      int r = idx / KC, kk = idx % KC;
      int e = e0 + r;
      ws[kk][r] = (e < E && kk < kn) ? load_f32(W, (int64_t)e * d + kc + kk) : 0.0f;
    }
    __syncthreads();
    for (int kk = 0; kk < kn; ++kk) {
      float a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = xs[kk][ty * TM + i];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = ws[kk][tx * TN + j];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int t = t0 + ty * TM + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int e = e0 + tx * TN + j;
      if (e >= E) continue;
      float s = sigmoid_fixed(acc[i][j]);
      s_out[(int64_t)t * E + e] = s;
      key_out[(int64_t)t * E + e] = __fadd_rn(s, bias[e]);
    }
  }
}

// Order-preserving map of an fp32 key to uint32 (larger key -> larger code);
// -0 and +0 map to the same code (they compare equal as floats).
__device__ __forceinline__ uint32_t key_code(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// One wave64 per token. Each lane holds NPER packed keys
// (code(key) << 32) | (0xFFFFFFFF - e): the maximum is the largest key, ties
// going to the lower expert index. k rounds of (lane max, wave max, retire);
// the wave maximum is the same on every lane, so lane j simply keeps the
// winner of round j. Gates: every lane forms the same slot-order sum of the
// chosen unbiased scores (broadcast one slot at a time), then slot j divides
// its own score by it. No block-level barrier: a wave past the last token
// just exits.
template <int NPER>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ s,
                                                   const float* __restrict__ key, int T,
                                                   int E, int k, int32_t* __restrict__ idx_out,
                                                   float* __restrict__ gate_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* kr = key + (int64_t)t * E;
  const float* sr = s + (int64_t)t * E;
  int32_t* ir = idx_out + (int64_t)t * k;
  float* gr = gate_out + (int64_t)t * k;

  uint64_t v[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    int e = lane + 64 * i;
    v[i] = (e < E) ? (((uint64_t)key_code(kr[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e))
                   : 0ull;
  }
  float total = 0.0f;
  for (int j0 = 0; j0 < k; j0 += 64) {
    const int jn = min(64, k - j0);
    int my_e = 0;
    for (int j = 0; j < jn; ++j) {
      uint64_t m = 0;
#pragma unroll
      for (int i = 0; i < NPER; ++i) m = v[i] > m ? v[i] : m;
      m = wave_max_u64(m);
      const int e = (int)(0xFFFFFFFFu - (uint32_t)m);
      if ((e & 63) == lane) {
#pragma unroll
        for (int i = 0; i < NPER; ++i)
          if (i == (e >> 6)) v[i] = 0ull;
      }
      if (lane == j) my_e = e;
    }
    const float my_s = (lane < jn) ? sr[my_e] : 0.0f;
    if (lane < jn) ir[j0 + lane] = my_e;
    for (int j = 0; j < jn; ++j) total = __fadd_rn(total, __shfl(my_s, j, 64));
  }
  // slot j = j0 + lane was written by this same lane above
  for (int j = lane; j < k; j += 64) gr[j] = __fdiv_rn(sr[ir[j]], total);
}

}  // namespace

template <int TMN, typename XT, typename WT>
void go_router(const RouterArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)ceil_div(a.E, 16 * TMN), (unsigned)ceil_div(a.T, 16 * TMN));
  hipLaunchKernelGGL((router_kernel<TMN, TMN, XT, WT>), grid, dim3(256), 0, stream,
                     (const XT*)a.x, (const WT*)a.W, a.bias, a.T, a.d, a.E, a.s, a.key);
}

// 8 x 8 micro-tiles (128 x 128 block) when the grid still fills the chip;
// 2 x 2 (32 x 32 block) for decode-sized batches.
int launch_router(const RouterArgs& a, hipStream_t stream) {
  if (a.T == 0) return 0;
  const bool big = (int64_t)a.T * a.E >= (int64_t)2048 * 896;
  if (a.x_dtype == DT_F32 && a.w_dtype == DT_F32) {
    if (big) go_router<8, float, float>(a, stream); else go_router<2, float, float>(a, stream);
  } else if (a.x_dtype == DT_BF16 && a.w_dtype == DT_BF16) {
    if (big) go_router<8, bf16_t, bf16_t>(a, stream); else go_router<2, bf16_t, bf16_t>(a, stream);
  } else {
    return -1;
  }
  return (int)hipGetLastError();
}

int launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.T == 0) return 0;
  dim3 grid((unsigned)ceil_div(a.T, 4));
  const int nper = (int)ceil_div(a.E, 64);
#define MOE_TOPK(N)                                                                           \
  hipLaunchKernelGGL(topk_kernel<N>, grid, dim3(256), 0, stream, a.s, a.key, a.T, a.E, a.k, \
                     a.idx, a.gate)
  if (nper <= 1) MOE_TOPK(1);
  else if (nper <= 2) MOE_TOPK(2);
  else if (nper <= 4) MOE_TOPK(4);
  else if (nper <= 8) MOE_TOPK(8);
  else if (nper <= 16) MOE_TOPK(16);
  else if (nper <= 32) MOE_TOPK(32);
  else if (nper <= 64) MOE_TOPK(64);
  else return -1;
#undef MOE_TOPK
  return (int)hipGetLastError();
}

}  // namespace moe
