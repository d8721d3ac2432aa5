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

// One DPP step of a 64-bit value: lane i gets the value of the lane that
// dpp control CTRL names within its row of 16 (every lane active).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Maximum over the wave (all 64 lanes active), the same value on every lane:
// within each row of 16 lanes by DPP (swap neighbours, swap pairs, mirror
// each half row, mirror the row: every lane then holds its row's maximum),
// then across the four rows from one lane of each.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xB1>(v));    // quad_perm [1, 0, 3, 2]
  v = max_u64(v, dpp_u64<0x4E>(v));    // quad_perm [2, 3, 0, 1]
  v = max_u64(v, dpp_u64<0x141>(v));   // row_half_mirror
  v = max_u64(v, dpp_u64<0x140>(v));   // row_mirror
  return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)),
                 max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

// A lane's two largest packed keys among its N slots (0: none; keys are
// unique), with the values that ride along; BELOW: only keys below `below`.
template <int N, bool S, bool BELOW>
__device__ __forceinline__ void top2_below(const uint64_t (&v)[N], const float (&sv)[N], uint64_t below,
                                           uint64_t& b1, float& s1, uint64_t& b2, float& s2) {
  b1 = 0ull; b2 = 0ull; s1 = 0.0f; s2 = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint64_t c = (!BELOW || v[i] < below) ? v[i] : 0ull;
    const bool gt1 = c > b1, gt2 = c > b2;   // selects, not branches (keeps b1, b2 in registers)
    b2 = gt1 ? b1 : gt2 ? c : b2;
    b1 = gt1 ? c : b1;
    if constexpr (S) {
      s2 = gt1 ? s1 : gt2 ? sv[i] : s2;
      s1 = gt1 ? sv[i] : s1;
    }
  }
}

// k rounds of "take the wave's largest key" over per-lane slots, without
// rescanning every slot each round: each lane keeps its two largest
// remaining keys (b1 > b2). The lane whose b1 is taken moves b2 up while b2
// is known to be its next key, and otherwise rescans its slots below the key
// just taken (every slot above it is gone: a lane gives up its keys in
// descending order). S: the value sv[i] rides along with key v[i]. Returns
// true on the lane that held m.
template <int N, bool S>
__device__ __forceinline__ bool walk_take(const uint64_t (&v)[N], const float (&sv)[N], uint64_t m,
                                          uint64_t& b1, float& s1, uint64_t& b2, float& s2,
                                          bool& next_known) {
  if (b1 != m) return false;   // m is held by exactly one lane's b1
  if (next_known) {
    b1 = b2; s1 = s2; b2 = 0ull; next_known = false;
  } else {
    top2_below<N, S, true>(v, sv, m, b1, s1, b2, s2);
    next_known = true;
  }
  return true;
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

// ---------------------------------------------------------------------------
// Matrix-core router with an exact recheck (bf16 x and W_r).
//
// The bf16 products x_k w_k are exact in fp32, so both the fixed fp32 chain
// and the matrix cores' fp32 accumulation are sums of the same d exact terms,
// each within gamma_d * sum_k |x_k w_k| <= gamma_d * |x| |w| of the exact sum
// (gamma_d = d u / (1 - d u), u = 2^-24, any summation order and rounding to
// nearest or toward zero at most doubles it). Hence the fixed-order logit lies
// in [L - beta, L + beta] with beta = 6 gamma_d |x_t| |w_e| for the matrix-core
// logit L. The sigmoid and "+ b_e" are monotone, so the fixed-order key lies in
// [key_lo, key_hi]. With L_k the k-th largest key_lo, any expert with
// key_hi < L_k is beaten by k experts and cannot be chosen: the candidates
// {e : key_hi >= L_k} hold the top-k. For them the fixed-order logit, sigmoid
// and key are computed exactly as the VALU router does, and the top-k and
// gates are taken among them: bit for bit the same result.
// ---------------------------------------------------------------------------

// Upper bounds of the row norms |A_r| (bf16 rows of K): the fp32 sum of
// squares is within gamma_K (about K 2^-24) of the exact one; the factor
// 1 + K 2^-22 covers that, and 1 + 2^-20 the rounding of the square root.
__global__ __launch_bounds__(256) void row_norms_kernel(const bf16_t* __restrict__ A, int rows, int K,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const bf16_t* row = A + (int64_t)r * K;
  float ss = 0.0f;
  for (int k = lane * 8; k < K; k += 64 * 8) {
    const uint4 v = *(const uint4*)(row + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __uint_as_float(w[j] << 16), hi = __uint_as_float(w[j] & 0xFFFF0000u);
      ss = __builtin_fmaf(lo, lo, ss);
      ss = __builtin_fmaf(hi, hi, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) out[r] = sqrtf(ss * (1.0f + (float)K * 0x1p-22f)) * (1.0f + 0x1p-20f);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One 64-thread block (one wave) per token; d % 64 == 0 and E d 2 < 2^31.
//  1. From the matrix-core logits: the interval [key_lo, key_hi] that holds
//     each expert's fixed-order key, and L_k, the k-th largest key_lo.
//  2. The candidates {e : key_hi >= L_k} (compacted in LDS), their fixed-order
//     logits 64 at a time, one per lane: the W rows of the 64 candidates pass
//     through LDS in chunks of KC k (coalesced loads of the next chunk run
//     while the lanes walk the current one); x goes to LDS widened to fp32.
//  3. The top-k of the exact keys (key descending, ties to the lower index)
//     and the gates s_j / sum_slots s, the sum in slot order.
// DIRECT (few tokens, one wave per CU, d % 256 == 0): step 2 keeps x in LDS
// as fp32 (dynamic shared memory, d floats) and each lane streams its own
// candidate's W row into registers, four 64-k chunks ahead; the FMA chain is
// the same. With no LDS staging of W there is no per-chunk wave sync, and the
// x reads are broadcasts.
template <int NPER, int KC, bool DIRECT = false>
__global__ __launch_bounds__(64) void select_kernel(SelectArgs a, float beta_coef) {
  constexpr int kChunk = KC;                 // k per staged chunk
  constexpr int kPPR = kChunk / 8;           // 16-byte pieces per W row per chunk
  constexpr int kRPL = 64 / kPPR;            // W rows per load instruction
  constexpr int kNJ = 64 / kRPL;             // load instructions per lane per chunk
  static_assert(kPPR <= 64 && 64 % kPPR == 0, "chunk");
  constexpr int kRowBytes = kChunk * 2 + 16; // LDS row stride (16 B pad: conflict-free reads)
  __shared__ int32_t cand_e[NPER * 64];
  __shared__ __align__(16) uint8_t wst[64 * kRowBytes];
  __shared__ __align__(16) float xst[kChunk];
  __shared__ float sel_s[64];
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  const float* Lr = a.L + (int64_t)t * a.E;
  const float xn = a.xn[t];

  // 1. interval keys; L_k
  uint64_t lo_code[NPER];
  float key_hi[NPER];
  // all loads first (index clamped into range, results of e >= E unused), so
  // their latencies overlap instead of adding up slot by slot
  float lv[NPER], wv[NPER], bv[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int ec = min(lane + 64 * i, a.E - 1);
    lv[i] = Lr[ec];
    wv[i] = a.wn[ec];
    bv[i] = a.bias[ec];
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    lo_code[i] = 0ull;
    key_hi[i] = -INFINITY;
    if (e < a.E) {
      const float l = lv[i];
      const float beta = beta_coef * xn * wv[i] + 1e-30f;
      const float s_lo = sigmoid_fixed(l - beta) * (1.0f - 0x1p-20f);
      const float s_hi = sigmoid_fixed(l + beta) * (1.0f + 0x1p-20f);
      const float b = bv[i];
      lo_code[i] = ((uint64_t)key_code(__fadd_rn(s_lo, b)) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
      key_hi[i] = __fadd_rn(s_hi, b);
    }
  }
  uint64_t kth = 0;
  {
    uint64_t b1, b2;
    float s1, s2;
    bool next_known = true;
    top2_below<NPER, false, false>(lo_code, key_hi, 0ull, b1, s1, b2, s2);   // no values ride along
    for (int j = 0; j < a.k; ++j) {
      kth = wave_max_u64(b1);
      walk_take<NPER, false>(lo_code, key_hi, kth, b1, s1, b2, s2, next_known);
    }
  }
  const uint32_t kc = (uint32_t)(kth >> 32);  // invert the order-preserving code of L_k
  const float Lk = __uint_as_float((kc & 0x80000000u) ? (kc & 0x7FFFFFFFu) : ~kc);

  // 2a. candidates, in expert order
  int ncand = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    const bool is_c = e < a.E && key_hi[i] >= Lk;
    const uint64_t mask = __ballot(is_c);
    if (is_c) cand_e[ncand + __popcll(mask & ((1ull << lane) - 1ull))] = e;
    ncand += __popcll(mask);
  }
  wave_sync();

  // 2b. fixed-order logits of the candidates; candidate p = 64 r + lane ends
  //     in code[r], sc[r] of this lane
  const rsrc_t xres = make_rsrc((const bf16_t*)a.x + (int64_t)t * a.d, (int64_t)a.d * 2);
  const int nchunks = a.d / kChunk;         // d % kChunk == 0 (checked by the launcher)
  uint64_t code[NPER];
  float sc[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) { code[i] = 0ull; sc[i] = 0.0f; }
  const int npass = (int)ceil_div(ncand, 64);
  if constexpr (DIRECT) {
    extern __shared__ __align__(16) float xs_dyn[];
    // x to LDS: a lane's 16-byte pieces (d / 512 of them) loaded 16 at a
    // time, all in flight before the first is widened
    constexpr int kXU = 16;
    for (int i0 = lane; i0 < a.d / 8; i0 += 64 * kXU) {
      uint4 xq[kXU];
#pragma unroll
      for (int u = 0; u < kXU; ++u) {
        const int i = i0 + 64 * u;
        xq[u] = bload16(xres, i < a.d / 8 ? (uint32_t)i * 16u : kOOB);
      }
#pragma unroll
      for (int u = 0; u < kXU; ++u) {
        const int i = i0 + 64 * u;
        if (i < a.d / 8) {
          const uint32_t xv[4] = {xq[u].x, xq[u].y, xq[u].z, xq[u].w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            xs_dyn[8 * i + 2 * m] = __uint_as_float(xv[m] << 16);
            xs_dyn[8 * i + 2 * m + 1] = __uint_as_float(xv[m] & 0xFFFF0000u);
          }
        }
      }
    }
    wave_sync();
    const int nch = a.d / 64;                // a multiple of 4 (d % 256 == 0)
    for (int r = 0; r < npass; ++r) {
      const int p = 64 * r + lane;
      const int ce = cand_e[p];              // in range: p < 64 NPER
      const uint32_t base = p < ncand ? (uint32_t)ce * (uint32_t)a.d * 2u : kOOB;
      uint4 q0[8], q1[8], q2[8], q3[8];
      // chunk c through a resource that starts c 64-k chunks into W (scalar
      // work only; a lane's offset is its row, or kOOB): past the row's end
      // (the prefetch beyond the last chunk) a lane reads the next row, or
      // zeros past W's end, and never uses what it read
      const int64_t wbytes = (int64_t)a.E * a.d * 2;
      auto load = [&](uint4 (&q)[8], int c) {
        const int64_t skip = 128 * (int64_t)c;
        const rsrc_t rc = make_rsrc((const uint8_t*)a.W + skip, wbytes > skip ? wbytes - skip : 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = bload16(rc, base + 16u * (uint32_t)j);
      };
      float acc = 0.0f;
      // scheduling barriers at each chunk (and between the first loads) keep
      // the widening of a chunk's W after the chunk before it and the loads in
      // chunk order, so that each chunk waits for its own loads only (left
      // free, the scheduler hoists all four chunks' widening to the loop top
      // and every round waits for every load in flight)
      auto chain = [&](uint4 (&q)[8], int c) {
        __builtin_amdgcn_sched_barrier(0);
        float4 xv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) xv[j] = *(const float4*)(xs_dyn + 64 * c + 4 * j);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float4 x0 = xv[2 * j], x1 = xv[2 * j + 1];
          const uint4 wv = q[j];
          acc = __builtin_fmaf(x0.x, __uint_as_float(wv.x << 16), acc);
          acc = __builtin_fmaf(x0.y, __uint_as_float(wv.x & 0xFFFF0000u), acc);
          acc = __builtin_fmaf(x0.z, __uint_as_float(wv.y << 16), acc);
          acc = __builtin_fmaf(x0.w, __uint_as_float(wv.y & 0xFFFF0000u), acc);
          acc = __builtin_fmaf(x1.x, __uint_as_float(wv.z << 16), acc);
          acc = __builtin_fmaf(x1.y, __uint_as_float(wv.z & 0xFFFF0000u), acc);
          acc = __builtin_fmaf(x1.z, __uint_as_float(wv.w << 16), acc);
          acc = __builtin_fmaf(x1.w, __uint_as_float(wv.w & 0xFFFF0000u), acc);
        }
        load(q, c + 4);
      };
      load(q0, 0);
      __builtin_amdgcn_sched_barrier(0);
      load(q1, 1);
      __builtin_amdgcn_sched_barrier(0);
      load(q2, 2);
      __builtin_amdgcn_sched_barrier(0);
      load(q3, 3);
      for (int c = 0; c < nch; c += 4) {
        chain(q0, c);
        chain(q1, c + 1);
        chain(q2, c + 2);
        chain(q3, c + 3);
      }
      if (p < ncand) {
        const float sv = sigmoid_fixed(acc);
        const uint64_t cd = ((uint64_t)key_code(__fadd_rn(sv, a.bias[ce])) << 32) |
                            (uint64_t)(0xFFFFFFFFu - (uint32_t)ce);
#pragma unroll
        for (int i = 0; i < NPER; ++i)
          if (i == r) { code[i] = cd; sc[i] = sv; }
      }
    }
  }
  for (int r = 0; r < (DIRECT ? 0 : npass); ++r) {
    // rows this lane loads: lane / kPPR + kRPL j, 16-byte piece lane % kPPR
    uint32_t roff[kNJ];
    int ce[kNJ];
#pragma unroll
    for (int j = 0; j < kNJ; ++j) ce[j] = cand_e[64 * r + lane / kPPR + kRPL * j];   // in range: p < 64 NPER
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      const int p = 64 * r + lane / kPPR + kRPL * j;
      roff[j] = p < ncand ? (uint32_t)ce[j] * (uint32_t)a.d * 2u + (uint32_t)(lane % kPPR) * 16u : kOOB;
    }
    const uint32_t xoff = lane < kPPR ? (uint32_t)lane * 16u : kOOB;
    uint4 pw[kNJ], px;
    // chunk c (< nchunks) through resources that start at its first k (scalar
    // work only; the lanes' offsets stay as they are)
    auto load_chunk = [&](int c) {
      const int64_t k0b = 2 * (int64_t)c * kChunk;
      const rsrc_t wc = make_rsrc((const uint8_t*)a.W + k0b, (int64_t)a.E * a.d * 2 - k0b);
      const rsrc_t xc = make_rsrc((const uint8_t*)a.x + (int64_t)t * a.d * 2 + k0b, (int64_t)a.d * 2 - k0b);
#pragma unroll
      for (int j = 0; j < kNJ; ++j) pw[j] = bload16(wc, roff[j]);
      px = bload16(xc, xoff);
    };
    load_chunk(0);
    float acc = 0.0f;
    for (int c = 0; c < nchunks; ++c) {
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
        *(uint4*)(wst + (lane / kPPR + kRPL * j) * kRowBytes + (lane % kPPR) * 16) = pw[j];
      if (lane < kPPR) {
        const uint32_t xv[4] = {px.x, px.y, px.z, px.w};
        float4 lo4, hi4;
        lo4.x = __uint_as_float(xv[0] << 16); lo4.y = __uint_as_float(xv[0] & 0xFFFF0000u);
        lo4.z = __uint_as_float(xv[1] << 16); lo4.w = __uint_as_float(xv[1] & 0xFFFF0000u);
        hi4.x = __uint_as_float(xv[2] << 16); hi4.y = __uint_as_float(xv[2] & 0xFFFF0000u);
        hi4.z = __uint_as_float(xv[3] << 16); hi4.w = __uint_as_float(xv[3] & 0xFFFF0000u);
        *(float4*)(xst + lane * 8) = lo4;
        *(float4*)(xst + lane * 8 + 4) = hi4;
      }
      wave_sync();
      if (c + 1 < nchunks) load_chunk(c + 1);
      const uint8_t* row = wst + lane * kRowBytes;
#pragma unroll
      for (int st = 0; st < kChunk / 8; ++st) {
        const uint4 wv = *(const uint4*)(row + st * 16);
        const float4 x0 = *(const float4*)(xst + st * 8);
        const float4 x1 = *(const float4*)(xst + st * 8 + 4);
        acc = __builtin_fmaf(x0.x, __uint_as_float(wv.x << 16), acc);
        acc = __builtin_fmaf(x0.y, __uint_as_float(wv.x & 0xFFFF0000u), acc);
        acc = __builtin_fmaf(x0.z, __uint_as_float(wv.y << 16), acc);
        acc = __builtin_fmaf(x0.w, __uint_as_float(wv.y & 0xFFFF0000u), acc);
        acc = __builtin_fmaf(x1.x, __uint_as_float(wv.z << 16), acc);
        acc = __builtin_fmaf(x1.y, __uint_as_float(wv.z & 0xFFFF0000u), acc);
        acc = __builtin_fmaf(x1.z, __uint_as_float(wv.w << 16), acc);
        acc = __builtin_fmaf(x1.w, __uint_as_float(wv.w & 0xFFFF0000u), acc);
      }
      wave_sync();
    }
    const int p = 64 * r + lane;
    if (p < ncand) {
      const int e = cand_e[p];
      const float sv = sigmoid_fixed(acc);
      const uint64_t cd = ((uint64_t)key_code(__fadd_rn(sv, a.bias[e])) << 32) |
                          (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (i == r) { code[i] = cd; sc[i] = sv; }
    }
  }

  // 3. top-k of the exact keys; gates
  int32_t* ir = a.idx + (int64_t)t * a.k;
  float* gr = a.gate + (int64_t)t * a.k;
  float total = 0.0f;
  uint64_t b1, b2;
  float s1, s2;
  bool next_known = true;
  top2_below<NPER, true, false>(code, sc, 0ull, b1, s1, b2, s2);
  float my_s = 0.0f;
  for (int j0 = 0; j0 < a.k; j0 += 64) {
    const int jn = min(64, a.k - j0);
    int my_e = 0;
    for (int j = 0; j < jn; ++j) {
      const uint64_t wmax = wave_max_u64(b1);
      const float s_taken = s1;
      if (wmax != 0ull && walk_take<NPER, true>(code, sc, wmax, b1, s1, b2, s2, next_known)) sel_s[j] = s_taken;
      if (lane == j) my_e = (int)(0xFFFFFFFFu - (uint32_t)wmax);
    }
    wave_sync();
    my_s = lane < jn ? sel_s[lane] : 0.0f;
    if (lane < jn) {
      ir[j0 + lane] = my_e;
      if (a.k > 64) gr[j0 + lane] = my_s;  // the score for now; divided by the sum below
    }
    for (int j = 0; j < jn; ++j) total = __fadd_rn(total, sel_s[j]);   // slot order
    wave_sync();
  }
  if (a.k <= 64) {
    if (lane < a.k) gr[lane] = __fdiv_rn(my_s, total);
  } else {
    // slot j was written by lane j % 64 above (the same thread reads it back)
    for (int j = lane; j < a.k; j += 64) gr[j] = __fdiv_rn(gr[j], total);
  }
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

int launch_row_norms(const void* A, int rows, int K, float* out, hipStream_t stream) {
  if (rows == 0) return 0;
  hipLaunchKernelGGL(row_norms_kernel, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, stream,
                     (const bf16_t*)A, rows, K, out);
  return (int)hipGetLastError();
}

bool router_select_supported(int E, int d) {
  return d % 64 == 0 && (int64_t)E * d * 2 < ((int64_t)1 << 31) && E <= 64 * 64;
}

int launch_router_select(const SelectArgs& a, hipStream_t stream) {
  if (a.T == 0) return 0;
  if (!router_select_supported(a.E, a.d)) return -1;
  // beta = 6 gamma_d |x| |w|: 4 gamma_d bounds the two sums' distance (rounding
  // to nearest or toward zero), the rest covers the fp32 evaluation of beta
  const double du = (double)a.d * 0x1p-24;
  const float beta_coef = (float)(6.0 * du / (1.0 - du));
  const int nper = (int)ceil_div(a.E, 64);
  // one wave per token: with fewer tokens than about 8 waves per CU the wave
  // has nothing to hide its latencies behind, so its candidates' W rows go
  // straight to registers several chunks ahead (x in dynamic LDS)
  const bool direct = a.T < 2048 && a.d % 256 == 0 && (size_t)a.d * 4 <= 96 * 1024;
  const size_t xs_bytes = direct ? (size_t)a.d * 4 : 0;
#define MOE_SEL(N)                                                                                    \
  do {                                                                                                \
    if (direct) hipLaunchKernelGGL((select_kernel<N, 64, true>), dim3((unsigned)a.T), dim3(64),        \
                                   xs_bytes, stream, a, beta_coef);                                   \
    else hipLaunchKernelGGL((select_kernel<N, 64>), dim3((unsigned)a.T), dim3(64), 0, stream, a,     \
                            beta_coef);                                                              \
  } while (0)
  if (nper <= 1) MOE_SEL(1);
  else if (nper <= 2) MOE_SEL(2);
  else if (nper <= 4) MOE_SEL(4);
  else if (nper <= 8) MOE_SEL(8);
  else if (nper <= 16) MOE_SEL(16);
  else if (nper <= 32) MOE_SEL(32);
  else if (nper <= 64) MOE_SEL(64);
  else return -1;
#undef MOE_SEL
  return (int)hipGetLastError();
}

}  // namespace moe
