// Token permutation: group the T*k (token, slot) pairs by expert.
//
// The flowchart on "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか"
// (lilting.ch, section "K3のエキスパートは896個の小型LLMではない") runs each token's
// 16 chosen expert FFNs; on one GPU that becomes: sort the (token, slot) pairs
// by expert so every expert's rows are contiguous for its grouped GEMM.
//
// Deterministic counting sort, no order decided by atomics:
//   1. hist:    per token-block LDS histogram  -> block_counts[b][e]
//   2. scan:    per expert, exclusive scan over blocks (block start inside the
//               expert's group); counts[e]; exclusive scan over experts ->
//               offsets; block starts += offsets[e]
//   3. scatter: one wave per token-block walks its tokens in order; slot j of
//               token t takes the next row of its expert. Within one token the
//               experts are distinct, so the LDS fetch-adds of one step touch
//               distinct counters and the order is fixed.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kPermTokens = 64;   // tokens per block in hist / scatter

__global__ __launch_bounds__(256) void perm_hist(const int32_t* __restrict__ idx, int T, int E,
                                                 int k, int32_t* __restrict__ block_counts) {
  extern __shared__ int32_t cnt[];
  for (int i = threadIdx.x; i < E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kPermTokens;
  const int t1 = min(T, t0 + kPermTokens);
  for (int64_t a = (int64_t)t0 * k + threadIdx.x; a < (int64_t)t1 * k; a += blockDim.x) {
    int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += blockDim.x)
    block_counts[(int64_t)blockIdx.x * E + i] = cnt[i];
}

// Exclusive scan of v[0..n) in LDS by one block of 1024 threads (n <= 4096).
__device__ void block_exclusive_scan(int32_t* v, int n, int32_t* part, int32_t* total) {
  const int tid = threadIdx.x;
  constexpr int PER = 4;
  int32_t loc[PER];
  int32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int j = tid * PER + i;
    loc[i] = (j < n) ? v[j] : 0;
    sum += loc[i];
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t add = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int32_t run = part[tid] - sum;  // exclusive prefix of this thread's chunk
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int j = tid * PER + i;
    if (j < n) v[j] = run;
    run += loc[i];
  }
  if (tid == 1023) *total = part[1023];
  __syncthreads();
}

__global__ __launch_bounds__(1024) void perm_scan(int32_t* __restrict__ block_counts, int nblk,
                                                  int E, int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets) {
  __shared__ int32_t sh[4096];
  __shared__ int32_t part[1024];
  __shared__ int32_t total;
  // a thread per expert walks the token blocks in order, kScanU blocks' counts
  // loaded at a time
  constexpr int kScanU = 16;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t run = 0;
    for (int b0 = 0; b0 < nblk; b0 += kScanU) {
      int32_t c[kScanU];
#pragma unroll
      for (int u = 0; u < kScanU; ++u) c[u] = b0 + u < nblk ? block_counts[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanU; ++u)
        if (b0 + u < nblk) {
          block_counts[(int64_t)(b0 + u) * E + e] = run;
          run += c[u];
        }
    }
    sh[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  block_exclusive_scan(sh, E, part, &total);
  for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = sh[e];
  if (threadIdx.x == 0) offsets[E] = total;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int32_t base = sh[e];
    for (int b0 = 0; b0 < nblk; b0 += kScanU) {
      int32_t c[kScanU];
#pragma unroll
      for (int u = 0; u < kScanU; ++u) c[u] = b0 + u < nblk ? block_counts[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanU; ++u)
        if (b0 + u < nblk) block_counts[(int64_t)(b0 + u) * E + e] = c[u] + base;
    }
  }
}

__global__ __launch_bounds__(256) void perm_scatter(const int32_t* __restrict__ idx, int T, int E,
                                                    int k, const int32_t* __restrict__ block_start,
                                                    int32_t* __restrict__ perm_src,
                                                    int32_t* __restrict__ inv_pos) {
  extern __shared__ int32_t pos[];
  for (int i = threadIdx.x; i < E; i += blockDim.x)
    pos[i] = block_start[(int64_t)blockIdx.x * E + i];
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int t0 = blockIdx.x * kPermTokens;
  const int t1 = min(T, t0 + kPermTokens);
  const auto place = [&](int64_t a, int e) {
    if (e >= 0 && e < E) {
      const int p = atomicAdd(&pos[e], 1);
      perm_src[p] = (int32_t)a;
      inv_pos[a] = p;
    } else {
      inv_pos[a] = -1;
    }
  };
  if (k <= 64) {
    // lane j < k takes slot j of every token. All of the block's expert ids
    // are loaded before the walk and every store waits until after it, so
    // the walk (in token order) waits on its LDS fetch-adds only.
    int32_t ev[kPermTokens], pv[kPermTokens];
#pragma unroll
    for (int i = 0; i < kPermTokens; ++i)
      ev[i] = (lane < k && t0 + i < t1) ? idx[(int64_t)(t0 + i) * k + lane] : -1;
#pragma unroll
    for (int i = 0; i < kPermTokens; ++i)
      pv[i] = (ev[i] >= 0 && ev[i] < E) ? atomicAdd(&pos[ev[i]], 1) : -1;
#pragma unroll
    for (int i = 0; i < kPermTokens; ++i)
      if (t0 + i < t1 && lane < k) {
        const int64_t a = (int64_t)(t0 + i) * k + lane;
        if (pv[i] >= 0) perm_src[pv[i]] = (int32_t)a;
        inv_pos[a] = pv[i];
      }
  } else {
    for (int t = t0; t < t1; ++t)
      for (int j = lane; j < k; j += 64) {
        const int64_t a = (int64_t)t * k + j;
        place(a, idx[a]);
      }
  }
}

__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ offsets, int E,
                                                          int BM, int32_t* __restrict__ tile_off,
                                                          int32_t* __restrict__ tile_info) {
  __shared__ int32_t sh[4096];
  __shared__ int32_t part[1024];
  __shared__ int32_t total;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t c = offsets[e + 1] - offsets[e];
    sh[e] = c > 0 ? (c + BM - 1) / BM : 0;
  }
  __syncthreads();
  block_exclusive_scan(sh, E, part, &total);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    tile_off[e] = sh[e];
    const int32_t o0 = offsets[e], c = offsets[e + 1] - o0;
    const int n = c > 0 ? (c + BM - 1) / BM : 0;
    for (int i = 0; i < n; ++i)
      *(int4*)(tile_info + 4 * (int64_t)(sh[e] + i)) = make_int4(e, sh[e], c, o0);
  }
  if (threadIdx.x == 0) tile_off[E] = total;
}

__global__ void fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

int permute_blocks(int T) { return (int)ceil_div(T, kPermTokens); }

int launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const int nblk = permute_blocks(a.T);
  const size_t lds = (size_t)a.E * sizeof(int32_t);
  if (a.T == 0) {
    // empty batch: zero counts and offsets (a fill kernel, not a memset node)
    hipLaunchKernelGGL(fill_i32, dim3(1), dim3(256), 0, stream, a.counts, (int64_t)a.E, 0);
    hipLaunchKernelGGL(fill_i32, dim3(1), dim3(256), 0, stream, a.offsets, (int64_t)a.E + 1, 0);
    return (int)hipGetLastError();
  }
  hipLaunchKernelGGL(perm_hist, dim3(nblk), dim3(256), lds, stream, a.idx, a.T, a.E, a.k,
                     a.block_counts);
  hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, stream, a.block_counts, nblk, a.E,
                     a.counts, a.offsets);
  hipLaunchKernelGGL(perm_scatter, dim3(nblk), dim3(256), lds, stream, a.idx, a.T, a.E, a.k,
                     a.block_counts, a.perm_src, a.inv_pos);
  return (int)hipGetLastError();
}

int launch_tile_table(const int32_t* offsets, int E, int BM, int32_t* tile_off, int32_t* tile_info,
                      hipStream_t stream) {
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, stream, offsets, E, BM, tile_off,
                     tile_info);
  return (int)hipGetLastError();
}

}  // namespace moe
