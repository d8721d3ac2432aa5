// Internal launchers of the gfx950 Stable LatentMoE kernels (not part of the ABI).
// Every launcher only enqueues on `stream`; it returns 0 or a hipError_t value
// (or -1 for an internal dispatch error). Shapes are checked by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RouterArgs {
  const void* x; int x_dtype;      // [T, d]
  const void* W; int w_dtype;      // [E, d]
  const float* bias;               // [E]
  int T, d, E;
  float* s;                        // [T, E]
  float* key;                      // [T, E]
};
int launch_router(const RouterArgs& a, hipStream_t stream);

// Router on the matrix cores with an exact recheck (bf16 x and W_r):
//   1. row norms of x and W_r (upper bounds, fp32)
//   2. approximate logits L = x W_r^T (bf16 MFMA, fp32 accumulate; split-K
//      partial sums added atomically: the values only bound the exact ones)
//   3. per token: interval keys from L +- beta, the candidate set that
//      provably holds the top-k, the fixed-order fp32 logit / sigmoid / key of
//      each candidate, and the exact top-k and gates.
int launch_row_norms(const void* A, int rows, int K, float* out, hipStream_t stream);
struct LogitsArgs {
  const void* x; const void* W;      // [T, d], [E, d] bf16
  int T, E, d;
  int splits;                        // K splits (atomic accumulation when > 1)
  float* L;                          // [T, E] fp32 (zeroed by the launcher when splits > 1)
};
int launch_router_logits(const LogitsArgs& a, hipStream_t stream);
int router_logit_splits(int T, int E, int d);
struct SelectArgs {
  const float* L;                    // [T, E] approximate logits
  const void* x; const void* W;      // [T, d], [E, d] bf16
  const float* bias;                 // [E]
  const float* xn; const float* wn;  // [T], [E] row norms
  int T, E, d, k;
  int32_t* idx; float* gate;         // [T, k]
};
int launch_router_select(const SelectArgs& a, hipStream_t stream);
bool router_select_supported(int E, int d);  // shapes the select kernel takes

struct TopkArgs {
  const float* s; const float* key;
  int T, E, k;
  int32_t* idx; float* gate;       // [T, k]
};
int launch_topk(const TopkArgs& a, hipStream_t stream);

// Permutation. Scratch: block_counts [nblk * E] int32 with nblk = permute_blocks(T).
int permute_blocks(int T);
struct PermuteArgs {
  const int32_t* idx; int T, E, k;
  int32_t* counts; int32_t* offsets; int32_t* perm_src; int32_t* inv_pos;
  int32_t* block_counts;
};
int launch_permute(const PermuteArgs& a, hipStream_t stream);

// Tile table of a grouped GEMM with BM-row tiles (device side, from offsets):
// tile_off[e] = sum_{e'<e} ceil(count_e' / BM), tile_off[E] = total tiles, and
// for each tile t of expert e, tile_info[4t .. 4t+3] = {e, tile_off[e],
// count_e, offsets[e]} (tile_info holds max_tiles entries).
int launch_tile_table(const int32_t* offsets, int E, int BM, int32_t* tile_off, int32_t* tile_info,
                      hipStream_t stream);

// A weight operand [rows, K] in bf16, fp32 or MXFP4 (data = packed, scale = e8m0).
struct WOperand {
  const void* data;
  const uint8_t* scale;
  int dtype;
};

// Split-K plan of a dense bf16 GEMM with few output rows: K is cut into
// `splits` ranges of `kchunk` (the last may be shorter); each (tile, range)
// block writes its fp32 partial tile to P[split][M][ncols], and a reduce kernel
// sums the splits in ascending order and applies the epilogue. splits == 0:
// the single-pass kernel (enough tiles to fill the chip; no partials).
struct SplitK {
  int splits = 0, kchunk = 0;
  int64_t partial_bytes(int64_t M, int64_t ncols) const { return (int64_t)splits * M * ncols * 4; }
};
SplitK plan_split(int act_dtype, int M, int ncols, int K);
// Partial slices of the output GEMM (one per segment) when it takes the split
// path, else 0.
int multiseg_slices(int act_dtype, int M, int N, int nseg);

// C[M, N] = A[M, K] W[N, K]^T, store in the act dtype. (latent down)
struct DenseArgs {
  const void* A; int64_t lda;  // act dtype
  WOperand W;                  // [N, K]
  int M, N, K;
  void* C; int64_t ldc;        // act dtype
  int act_dtype;
  SplitK split;                // plan_split(act_dtype, M, N, K)
  float* P;                    // split.partial_bytes(M, N) bytes when split.splits > 0
};
// The split form reads bf16 or MXFP4 W; the single pass (split.splits == 0)
// bf16 W only (an MXFP4 weight is decoded with launch_decode_mxfp4 first).
int launch_dense(const DenseArgs& a, hipStream_t stream);
// out[rows, K] bf16 = the exact values of the row-major MXFP4 weight w
// (packed [rows, K/2], scales [rows, K/32]; K % 32 == 0).
int launch_decode_mxfp4(const WOperand& w, int64_t rows, int K, void* out, hipStream_t stream);

// H[M, F] = act(A Wg^T, A Wv^T), Wg/Wv [F, K]. (shared gate/up)
struct GluArgs {
  const void* A; int64_t lda;
  WOperand Wg, Wv;
  int M, F, K;
  void* H; int64_t ldh;
  float c;
  int act_dtype;
  SplitK split;                // plan_split(act_dtype, M, 2 F, K)
  float* P;                    // split.partial_bytes(M, 2 F) bytes when split.splits > 0
};
int launch_glu(const GluArgs& a, hipStream_t stream);   // bf16 Wg, Wv only

// Grouped over experts: rows r in [offsets[e], offsets[e+1]) of expert e.
// gate/up: A row = z[perm_src[r] / k]; H[r] = act(z Wg[e]^T, z Wv[e]^T).
struct GroupedGluArgs {
  const void* Z; int64_t ldz;        // [T, K]
  int T;                             // rows of Z
  int rows_cap;                      // rows of H (T*k): rows at or past it are skipped
  const int32_t* perm_src; int topk;
  const int32_t* offsets;            // [E+1]
  const int32_t* tile_off;           // [E+1] for BM-row tiles
  const int32_t* tile_info;          // [max_tiles][4] (launch_tile_table)
  int max_tiles;                     // upper bound of tile_off[E]
  WOperand Wg, Wv;                   // [E, F, K]
  int E, F, K;
  void* H;                           // [rows, F]
  float c;
  int act_dtype;
  int bm;                            // tile rows (grouped_bm)
  int act_mx8;                       // Z holds MXFP8 codes ([T, K] bytes, row stride ldz
                                     // bytes) with scales z_scale [T, K/32]: scaled MFMA
  const uint8_t* z_scale;
  int w_tiled;                       // Wg / Wv tiled: MXFP4 with act_mx8 (launch_tile_mxfp4),
                                     // or bf16 (launch_tile_bf16)
  uint8_t* hq;                       // act_mx8 only: with hq (and hqs) set, h goes out as
  uint8_t* hqs;                      // MXFP8 codes [rows, F] and scales [rows, F/32];
                                     // else to bf16 H (one of the two must be given)
};
int launch_grouped_glu(const GroupedGluArgs& a, hipStream_t stream);
// Tile rows of the grouped expert kernels for `rows` routed rows over E
// experts: 1 (fp32 path), 128 or 256 (the LDS-tiled MFMA kernels; the launchers
// take the kernel that matches).
int grouped_bm(int act_dtype, int expert_w_dtype, int act_mx8, int w_tiled, int64_t rows, int E);
// Fragment-tiled copy of a bf16 weight [rows, K] (rows % 32 == 0, K % 8 == 0)
// for the grouped expert kernels that keep the weights in registers: for each
// group g of 32 rows and k-step s of 16 (K padded with zeros to Kp, the next
// multiple of 64), the 1 KB at (g (Kp/16) + s) 1024 holds 64 lanes x 8 bf16,
// lane l = row 32 g + l % 32, k = 16 s + 8 (l / 32) .. +7. tiled_bf16_bytes:
// the size of that copy.
int launch_tile_bf16(const void* in, void* out, int64_t rows, int K, hipStream_t stream);
int64_t tiled_bf16_bytes(int64_t rows, int K);
// Fragment-tiled copy of a row-major MXFP4 weight (rows % 32 == 0, K % 32 ==
// 0) for the same kernels, decoded in registers: K padded to Kp (the next
// multiple of 128) with zeros; packed codes: per group g of 32 rows and 64-k
// tile t, the 1 KB at (g (Kp/64) + t) 1024 holds 64 lanes x 16 bytes, lane l
// (row 32 g + l % 32) with the 8 codes of k = 64 t + 16 s + 8 (l / 32) .. +7 in
// its dword s; scales: per group g and 128-k pair p, the 128 bytes at
// (g (Kp/128) + p) 128 hold 32 rows x the 4 scale bytes of k-blocks 4p .. 4p+3.
int launch_tile_mxfp4_frag(const uint8_t* data, const uint8_t* scale, uint8_t* data_out, uint8_t* scale_out,
                           int64_t rows, int K, hipStream_t stream);
void tiled_mxfp4_frag_bytes(int64_t rows, int K, int64_t* data_bytes, int64_t* scale_bytes);

// down: O[r] = H[r] Wo[e]^T, Wo [E, N, K].
struct GroupedDownArgs {
  const void* H; int64_t ldh;
  int rows_cap;                      // rows of H and O
  const int32_t* offsets;
  const int32_t* tile_off;
  const int32_t* tile_info;
  int max_tiles;
  WOperand Wo;
  int E, N, K;
  void* O;
  int act_dtype;
  int bm;                            // tile rows (grouped_bm)
  int act_mx8;                       // H holds MXFP8 codes ([rows, K] bytes, row stride
                                     // ldh bytes) with scales h_scale [rows, K/32]
  const uint8_t* h_scale;
  int w_tiled;                       // Wo tiled (as GroupedGluArgs::w_tiled)
};
// MXFP8 (E4M3 + e8m0 per 32) rows of a bf16 matrix [rows, K] (row stride ld
// elements; K % 32 == 0): codes [rows, K], scales [rows, K/32] (OCP MX rule:
// X = floor(log2 amax) - 8, elements rounded to nearest even, saturating).
int launch_quantize_mx8(const void* in, int64_t rows, int K, int64_t ld, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream);
// Tiled copy of a row-major MXFP4 weight [rows, K] (rows % 64 == 0, K % 128
// == 0) for the scaled-MFMA kernels: packed byte j (0..63) of row r's stage kt
// (bytes 64kt .. 64kt+63 of the row) goes to ((r/2)(K/128) + kt) 128 +
// (r%2) 64 + j; scale byte (r, b) goes to ((r/64)(K/128) + b/4) 256 + (r%64) 4
// + b%4.
int launch_tile_mxfp4(const uint8_t* data, const uint8_t* scale, uint8_t* data_out, uint8_t* scale_out,
                      int64_t rows, int K, hipStream_t stream);
int launch_grouped_down(const GroupedDownArgs& a, hipStream_t stream);

// y[M, N] = sum over segments s of A_s[M, K_s] B_s[N, K_s]^T (fp32 accumulate).
struct Segment {
  const void* A; int64_t lda;
  WOperand B;
  int K;
};
constexpr int kMaxSegments = 8;
struct MultiSegArgs {
  Segment seg[kMaxSegments];
  int nseg;
  int M, N;
  void* C; int64_t ldc;
  int act_dtype;
  float* P;                    // multiseg_slices(...) * M * N fp32 when that is > 0
};
// Only the last segment's B may be MXFP4, and then only in the split form
// (multiseg_slices(...) > 0); the single pass takes bf16 B in every segment.
int launch_multiseg(const MultiSegArgs& a, hipStream_t stream);
// The split form in two parts (only when multiseg_slices(...) > 0): the fp32
// partial products of segments s0 .. s0 + ns - 1 into P[s] (each segment's
// own slice), then the ordered sum of all slices into C. launch_multiseg is
// partials(0, nseg) followed by reduce; the parts may run on different
// streams (the caller orders them).
int launch_multiseg_partials(const MultiSegArgs& a, int s0, int ns, hipStream_t stream);
int launch_multiseg_reduce(const MultiSegArgs& a, hipStream_t stream);

// fp32-activation variants of the GEMM launchers (gemm_f32.hip).
int launch_dense_f32(const DenseArgs& a, hipStream_t stream);
int launch_glu_f32(const GluArgs& a, hipStream_t stream);
int launch_grouped_glu_f32(const GroupedGluArgs& a, hipStream_t stream);
int launch_grouped_down_f32(const GroupedDownArgs& a, hipStream_t stream);
int launch_multiseg_f32(const MultiSegArgs& a, hipStream_t stream);

// Quantile Balancing bias: q[e] = the c-th largest scores[t][e] over t with
// c = qb_target(T, E, k); bias[e] = fp32(tau - q[e]), tau = fp32(mean of q)
// (fp64 sum, e ascending). T > 0.
int qb_target(int T, int E, int k);
int launch_qb_bias(const float* scores, int T, int E, int k, float* q, float* bias,
                   hipStream_t stream);

// Combine + RMSNorm.
struct CombineArgs {
  const void* O;                 // [T*k, D] act dtype, permuted rows
  const int32_t* inv_pos;        // [T*k]
  const float* gate;             // [T, k]
  const float* gain;             // [D] or null
  int T, k, D;
  float eps;
  void* n_out; int64_t ldn;      // [T, D] act dtype
  float* u_out;                  // [T, D] or null
  int act_dtype;
};
int launch_combine(const CombineArgs& a, hipStream_t stream);

}  // namespace moe
