// Matrix-core GEMMs of the Stable LatentMoE layer (gfx950, bf16 MFMA).
//
// Equations on "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか"
// (lilting.ch, section "K3のエキスパートは896個の小型LLMではない"):
//   z = W_down x                       -> dense   (latent down)
//   E_i(z) = W_o act(W_g z, W_v z)     -> grouped_glu + grouped_down (routed experts)
//   E_s(x)                             -> glu (shared gate/up) + multiseg
//   y = sum_s E_s(x) + W_up RMSNorm(u) -> multiseg: one GEMM whose K runs over the
//                                          shared experts' down projections and
//                                          then over W_up (sums over experts are
//                                          concatenations along K)
// Activation SiTU-GLU ("Kimi K3 テクニカルレポート", jiwasawa.github.io, section
// "幅のスケーリング: Stable LatentMoE"): act(g, v) = c tanh(SiLU(g)/c) c tanh(v/c).
// MXFP4 weights ("Kimi K3 ... Open Frontier Intelligence", ai-tech-express.jp,
// section "MXFP4 Quantization-Aware Training") are decoded to bf16 while they
// are staged into LDS; decoding is exact, so the MFMA itself stays bf16.
//
// Engine (bf16): block tile 128 x 128 x 64, 256 threads = 4 wave64 in a 2 x 2
// grid, each wave 64 x 64 = 2 x 2 tiles of v_mfma_f32_32x32x16_bf16, fp32
// accumulators. Operands are staged global -> registers -> LDS (row stride 72
// bf16: 16-byte reads of 8 consecutive rows hit distinct banks), double
// buffered: the next K-tile's global loads are in flight while the MFMAs run.
// Every weight row is K-contiguous ([out, in] layout), so A and B tiles are
// both "rows x K" and load the same way.
//
// fp32 activations (the small fp32 layer) use plain one-thread-per-output
// kernels: that layer is a parity case, not a throughput target.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;                         // LDS row stride (bf16 elements)
constexpr int STAGE = (BM + BN) * LDK;              // elements per pipeline stage
constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(bf16_t);

// ---------------------------------------------------------------------------
// operand staging
// ---------------------------------------------------------------------------

// This thread's share of a 128-row x 64-k bf16 tile: rows r0 + 32 i (i < 4),
// k-chunk kc (8 elements = 16 bytes); 8 consecutive threads cover one row's
// 128 bytes.
struct RowSet {
  const bf16_t* row[4];  // start of each row in global memory (nullptr: zero row)
};

__device__ __forceinline__ void load_rows(const RowSet& rs, int kc, int k0, int K, uint4 (&v)[4]) {
  const int k = k0 + kc * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (rs.row[i] != nullptr && k < K) v[i] = *(const uint4*)(rs.row[i] + k);
    else v[i] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_rows(bf16_t* tile, int r0, int kc, const uint4 (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *(uint4*)(tile + (r0 + 32 * i) * LDK + kc * 8) = v[i];
}

// MXFP4 rows: this thread owns one (row, 32-element half) unit of the
// 128-row x 64-k tile: row = tid / 2, half = tid % 2.
struct MxRow {
  const uint8_t* packed;  // row start (K/2 bytes), nullptr: zero row
  const uint8_t* scale;   // row start (K/32 bytes)
};

struct MxStage {
  uint4 q;       // 32 e2m1 codes
  uint32_t s;    // e8m0 scale byte (256 = zero block)
};

__device__ __forceinline__ void load_mx(const MxRow& m, int half, int k0, int K, MxStage& st) {
  const int k = k0 + half * 32;
  if (m.packed != nullptr && k < K) {
    st.q = *(const uint4*)(m.packed + k / 2);
    st.s = m.scale[k / 32];
  } else {
    st.q = make_uint4(0, 0, 0, 0);
    st.s = 256;
  }
}

// e2m1 code (4 bits) -> bf16 bits of its value (OCP MX: 0, .5, 1, 1.5, 2, 3, 4, 6).
__device__ __forceinline__ uint32_t e2m1_bf16(uint32_t c) {
  uint32_t m = c & 7u;
  uint32_t b = (m >= 2u) ? (0x3F80u + ((m - 2u) << 6)) : (m == 1u ? 0x3F00u : 0u);
  return b | ((c & 8u) << 12);
}

// value * 2^(s-127) exactly (power-of-two scaling of a 2-significant-bit value).
__device__ __forceinline__ uint32_t scale_bf16(uint32_t b, float scale) {
  float v = __uint_as_float(b << 16) * scale;
  return __float_as_uint(v) >> 16;
}

__device__ __forceinline__ void store_mx(bf16_t* tile, int row, int half, const MxStage& st) {
  uint32_t w[16];
  if (st.s == 256u) {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = 0;
  } else {
    const float scale = st.s == 0u ? 0x1p-127f : __uint_as_float(st.s << 23);
    const uint32_t q[4] = {st.q.x, st.q.y, st.q.z, st.q.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t byte = (q[i / 4] >> (8 * (i % 4))) & 0xFFu;
      const uint32_t lo = scale_bf16(e2m1_bf16(byte & 0xFu), scale);
      const uint32_t hi = scale_bf16(e2m1_bf16(byte >> 4), scale);
      w[i] = lo | (hi << 16);
    }
  }
  bf16_t* dst = tile + row * LDK + half * 32;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *(uint4*)(dst + 8 * i) = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
}

// ---------------------------------------------------------------------------
// the MFMA main loop over one K range
// ---------------------------------------------------------------------------

struct Acc {
  f32x16 c[2][2];
};

__device__ __forceinline__ void acc_zero(Acc& acc) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.c[i][j][r] = 0.0f;
}

__device__ __forceinline__ void mma_stage(const bf16_t* As, const bf16_t* Bs, int wm, int wn,
                                          int lane, Acc& acc) {
  const int lr = lane & 31, lk = (lane >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = *(const bf16x8*)(As + (wm * 64 + i * 32 + lr) * LDK + ks * 16 + lk);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *(const bf16x8*)(Bs + (wn * 64 + j * 32 + lr) * LDK + ks * 16 + lk);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.c[i][j], 0, 0, 0);
  }
}

// acc += A_tile(rows of `ar`) * B_tile(rows of `br` / `bm`)^T over k in [0, K).
template <bool B_MX>
__device__ void mainloop(bf16_t* lds, const RowSet& ar, const RowSet& br, const MxRow& bm, int K,
                         Acc& acc) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int r0 = tid >> 3, kc = tid & 7;
  const int mrow = tid >> 1, mhalf = tid & 1;
  const int nk = (int)ceil_div(K, BK);

  uint4 va[4], vb[4];
  MxStage mx;
  load_rows(ar, kc, 0, K, va);
  if constexpr (B_MX) load_mx(bm, mhalf, 0, K, mx); else load_rows(br, kc, 0, K, vb);
  store_rows(lds, r0, kc, va);
  if constexpr (B_MX) store_mx(lds + BM * LDK, mrow, mhalf, mx);
  else store_rows(lds + BM * LDK, r0, kc, vb);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    bf16_t* cur = lds + (kt & 1) * STAGE;
    bf16_t* nxt = lds + ((kt + 1) & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      load_rows(ar, kc, (kt + 1) * BK, K, va);
      if constexpr (B_MX) load_mx(bm, mhalf, (kt + 1) * BK, K, mx);
      else load_rows(br, kc, (kt + 1) * BK, K, vb);
    }
    mma_stage(cur, cur + BM * LDK, wm, wn, lane, acc);
    if (more) {
      store_rows(nxt, r0, kc, va);
      if constexpr (B_MX) store_mx(nxt + BM * LDK, mrow, mhalf, mx);
      else store_rows(nxt + BM * LDK, r0, kc, vb);
    }
    __syncthreads();
  }
}

// Element (i, j, r) of this lane's accumulators sits at tile row / column:
//   row = wm*64 + i*32 + 8*(r/4) + 4*(lane/32) + r%4,  col = wn*64 + j*32 + lane%32.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * 64 + j * 32 + (lane & 31); }

// Row set for B rows n0 + tile_row of a [N, K] bf16 matrix (rows >= N: zero).
__device__ __forceinline__ RowSet b_rows_plain(const bf16_t* W, int64_t ldw, int n0, int N) {
  RowSet rs;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int n = n0 + r0 + 32 * i;
    rs.row[i] = n < N ? W + (int64_t)n * ldw : nullptr;
  }
  return rs;
}

__device__ __forceinline__ MxRow b_mx_plain(const uint8_t* P, const uint8_t* S, int K, int n0, int N) {
  MxRow m;
  int n = n0 + (threadIdx.x >> 1);
  m.packed = n < N ? P + (int64_t)n * (K / 2) : nullptr;
  m.scale = n < N ? S + (int64_t)n * (K / 32) : nullptr;
  return m;
}

// GLU B tile: wave column wn covers tile rows wn*64 .. +63 = gate rows f0 + wn*32 + (0..31)
// then up rows f0 + wn*32 + (0..31).
__device__ __forceinline__ void glu_row_of(int tile_row, int f0, int& f, bool& up) {
  const int wn = tile_row >> 6, w = tile_row & 63;
  up = w >= 32;
  f = f0 + wn * 32 + (w & 31);
}

__device__ __forceinline__ RowSet b_rows_glu(const bf16_t* Wg, const bf16_t* Wv, int64_t ldw, int f0,
                                             int F) {
  RowSet rs;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int f;
    bool up;
    glu_row_of(r0 + 32 * i, f0, f, up);
    rs.row[i] = f < F ? (up ? Wv : Wg) + (int64_t)f * ldw : nullptr;
  }
  return rs;
}

__device__ __forceinline__ MxRow b_mx_glu(const WOperand& g, const WOperand& v, int64_t row_base,
                                          int K, int f0, int F) {
  int f;
  bool up;
  glu_row_of(threadIdx.x >> 1, f0, f, up);
  MxRow m;
  const WOperand& w = up ? v : g;
  m.packed = f < F ? (const uint8_t*)w.data + (row_base + f) * (K / 2) : nullptr;
  m.scale = f < F ? w.scale + (row_base + f) * (K / 32) : nullptr;
  return m;
}

template <typename OT>
__device__ __forceinline__ void store_tile(const Acc& acc, OT* C, int64_t ldc, int m0, int n0, int M,
                                           int N) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, wm = wv >> 1, wn = wv & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + acc_col(wn, j, lane);
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + acc_row(wm, i, r, lane);
        if (m < M) store_f32(C, (int64_t)m * ldc + n, acc.c[i][j][r]);
      }
    }
}

// rows: output row index of tile row (m0 + tr) is out_row(tr) (or < 0: skip)
template <typename OT, typename RowMap>
__device__ __forceinline__ void store_glu(const Acc& acc, OT* H, int64_t ldh, int f0, int F, float c,
                                          RowMap out_row) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, wm = wv >> 1, wn = wv & 1;
  const float inv_c = 1.0f / c;
  const int f = f0 + wn * 32 + (lane & 31);
  if (f >= F) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t orow = out_row(acc_row(wm, i, r, lane));
      if (orow < 0) continue;
      store_f32(H, orow * ldh + f, situ_glu(acc.c[i][0][r], acc.c[i][1][r], c, inv_c));
    }
}

// ---------------------------------------------------------------------------
// kernels (bf16 activations)
// ---------------------------------------------------------------------------

template <bool B_MX>
__global__ __launch_bounds__(256) void dense_kernel(DenseArgs a) {
  extern __shared__ __align__(16) bf16_t lds[];
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  RowSet ar;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + r0 + 32 * i;
    ar.row[i] = m < a.M ? (const bf16_t*)a.A + (int64_t)m * a.lda : nullptr;
  }
  RowSet br{};
  MxRow bm{};
  if constexpr (B_MX) bm = b_mx_plain((const uint8_t*)a.W.data, a.W.scale, a.K, n0, a.N);
  else br = b_rows_plain((const bf16_t*)a.W.data, a.K, n0, a.N);
  Acc acc;
  acc_zero(acc);
  mainloop<B_MX>(lds, ar, br, bm, a.K, acc);
  store_tile(acc, (bf16_t*)a.C, a.ldc, m0, n0, a.M, a.N);
}

template <bool B_MX>
__global__ __launch_bounds__(256) void glu_kernel(GluArgs a) {
  extern __shared__ __align__(16) bf16_t lds[];
  const int m0 = blockIdx.y * BM, f0 = blockIdx.x * (BN / 2);
  RowSet ar;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + r0 + 32 * i;
    ar.row[i] = m < a.M ? (const bf16_t*)a.A + (int64_t)m * a.lda : nullptr;
  }
  RowSet br{};
  MxRow bm{};
  if constexpr (B_MX) bm = b_mx_glu(a.Wg, a.Wv, 0, a.K, f0, a.F);
  else br = b_rows_glu((const bf16_t*)a.Wg.data, (const bf16_t*)a.Wv.data, a.K, f0, a.F);
  Acc acc;
  acc_zero(acc);
  mainloop<B_MX>(lds, ar, br, bm, a.K, acc);
  const int M = a.M;
  store_glu(acc, (bf16_t*)a.H, a.ldh, f0, a.F, a.c,
            [=](int tr) -> int64_t { return m0 + tr < M ? (int64_t)(m0 + tr) : -1; });
}

// Which expert owns grouped tile `tile`: the e with tile_off[e] <= tile < tile_off[e+1].
__device__ __forceinline__ int expert_of_tile(const int32_t* tile_off, int E, int tile) {
  int lo = 0, hi = E;  // invariant: tile_off[lo] <= tile < tile_off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

template <bool B_MX>
__global__ __launch_bounds__(256) void grouped_glu_kernel(GroupedGluArgs a) {
  extern __shared__ __align__(16) bf16_t lds[];
  const int tile = blockIdx.y;
  if (tile >= a.tile_off[a.E]) return;
  const int e = expert_of_tile(a.tile_off, a.E, tile);
  const int row_lo = a.offsets[e] + (tile - a.tile_off[e]) * BM;
  const int row_hi = min(min(a.offsets[e + 1], row_lo + BM), a.rows_cap);
  const int f0 = blockIdx.x * (BN / 2);
  RowSet ar;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = row_lo + r0 + 32 * i;
    const bf16_t* p = nullptr;
    if (r >= 0 && r < row_hi) {
      const int src = a.perm_src[r];
      const int t = src / a.topk;
      if (src >= 0 && t < a.T) p = (const bf16_t*)a.Z + (int64_t)t * a.ldz;
    }
    ar.row[i] = p;
  }
  RowSet br{};
  MxRow bm{};
  const int64_t wrow = (int64_t)e * a.F;
  if constexpr (B_MX) {
    bm = b_mx_glu(a.Wg, a.Wv, wrow, a.K, f0, a.F);
  } else {
    br = b_rows_glu((const bf16_t*)a.Wg.data + wrow * a.K, (const bf16_t*)a.Wv.data + wrow * a.K,
                    a.K, f0, a.F);
  }
  Acc acc;
  acc_zero(acc);
  mainloop<B_MX>(lds, ar, br, bm, a.K, acc);
  store_glu(acc, (bf16_t*)a.H, a.F, f0, a.F, a.c,
            [=](int tr) -> int64_t {
              const int r = row_lo + tr;
              return (r >= 0 && r < row_hi) ? (int64_t)r : -1;
            });
}

template <bool B_MX>
__global__ __launch_bounds__(256) void grouped_down_kernel(GroupedDownArgs a) {
  extern __shared__ __align__(16) bf16_t lds[];
  const int tile = blockIdx.y;
  if (tile >= a.tile_off[a.E]) return;
  const int e = expert_of_tile(a.tile_off, a.E, tile);
  const int row_lo = a.offsets[e] + (tile - a.tile_off[e]) * BM;
  const int row_hi = min(min(a.offsets[e + 1], row_lo + BM), a.rows_cap);
  const int n0 = blockIdx.x * BN;
  RowSet ar;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = row_lo + r0 + 32 * i;
    ar.row[i] = (r >= 0 && r < row_hi) ? (const bf16_t*)a.H + (int64_t)r * a.ldh : nullptr;
  }
  RowSet br{};
  MxRow bm{};
  const int64_t wrow = (int64_t)e * a.N;
  if constexpr (B_MX) {
    bm = b_mx_plain((const uint8_t*)a.Wo.data + wrow * (a.K / 2), a.Wo.scale + wrow * (a.K / 32),
                    a.K, n0, a.N);
  } else {
    br = b_rows_plain((const bf16_t*)a.Wo.data + wrow * a.K, a.K, n0, a.N);
  }
  Acc acc;
  acc_zero(acc);
  mainloop<B_MX>(lds, ar, br, bm, a.K, acc);
  // rows row_lo.. of O (ld = N)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, wm = wv >> 1, wn = wv & 1;
  bf16_t* O = (bf16_t*)a.O;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + acc_col(wn, j, lane);
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_lo + acc_row(wm, i, r, lane);
        if (row >= 0 && row < row_hi) O[(int64_t)row * a.N + n] = f32_to_bf16(acc.c[i][j][r]);
      }
    }
}

// Segments are visited in order; each segment's B is bf16 or MXFP4.
__global__ __launch_bounds__(256) void multiseg_kernel(MultiSegArgs a) {
  extern __shared__ __align__(16) bf16_t lds[];
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  Acc acc;
  acc_zero(acc);
  const int r0 = threadIdx.x >> 3;
  for (int s = 0; s < a.nseg; ++s) {
    const Segment& sg = a.seg[s];
    RowSet ar;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int m = m0 + r0 + 32 * i;
      ar.row[i] = m < a.M ? (const bf16_t*)sg.A + (int64_t)m * sg.lda : nullptr;
    }
    if (sg.B.dtype == DT_MXFP4) {
      MxRow bm = b_mx_plain((const uint8_t*)sg.B.data, sg.B.scale, sg.K, n0, a.N);
      RowSet br{};
      mainloop<true>(lds, ar, br, bm, sg.K, acc);
    } else {
      RowSet br = b_rows_plain((const bf16_t*)sg.B.data, sg.K, n0, a.N);
      MxRow bm{};
      mainloop<false>(lds, ar, br, bm, sg.K, acc);
    }
  }
  store_tile(acc, (bf16_t*)a.C, a.ldc, m0, n0, a.M, a.N);
}

// ---------------------------------------------------------------------------
// weight-streaming grouped kernels (few rows per expert, e.g. decode)
//
// With ~5 rows per expert the expert GEMMs are bound by reading each touched
// expert's weights from HBM once. A block owns one expert tile of up to 32
// rows (two 16-row v_mfma_f32_16x16x32_bf16 tiles) and 64 weight rows (four
// 16-column tiles: for gate/up two gate + the two matching up tiles), and the
// four waves split K: each wave streams its quarter of the 64 weight rows
// straight from global memory into MFMA operand registers (no LDS staging;
// the next 64-k chunk is in flight while the current one is multiplied), and
// the partial sums are reduced through LDS in a fixed wave order.
//
// k assignment inside a 64-k chunk: lane group g = lane/16 takes k = g*16 ..
// g*16+15, 8 per MFMA step. A and B use the same assignment, so every MFMA
// still sums over its 32 k values, and the 4 lanes of a weight row read the
// row's whole 128-byte segment.
// ---------------------------------------------------------------------------

constexpr int SK_BM = 32;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 zero_frag() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ bf16x8 ld_frag(const bf16_t* row, int k, int K) {
  if (row == nullptr || k >= K) return zero_frag();
  return *(const bf16x8*)(row + k);
}

// 8 MXFP4 elements k..k+7 (k a multiple of 8) of one packed row, decoded to bf16.
__device__ __forceinline__ bf16x8 ld_frag_mx(const uint8_t* prow, const uint8_t* srow, int k, int K) {
  if (prow == nullptr || k >= K) return zero_frag();
  const uint32_t q = *(const uint32_t*)(prow + k / 2);
  const uint32_t sb = srow[k / 32];
  const float scale = sb == 0u ? 0x1p-127f : __uint_as_float(sb << 23);
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t byte = (q >> (8 * i)) & 0xFFu;
    w[i] = scale_bf16(e2m1_bf16(byte & 0xFu), scale) | (scale_bf16(e2m1_bf16(byte >> 4), scale) << 16);
  }
  return __builtin_bit_cast(bf16x8, w);
}

struct SkRows {
  const bf16_t* a[2];      // A rows of m-tiles 0, 1 (nullptr: zero row)
  const void* b[4];        // B rows of n-tiles 0..3 (bf16 row, or packed MXFP4 row)
  const uint8_t* bs[4];    // MXFP4 scale rows
};

struct SkFrag {
  bf16x8 a[2][2];          // [m][step]
  bf16x8 b[4][2];          // [n][step]
};

template <bool MX>
__device__ __forceinline__ void sk_load(const SkRows& r, int k0, int K, SkFrag& f) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int k = k0 + g * 16 + st * 8;
#pragma unroll
    for (int m = 0; m < 2; ++m) f.a[m][st] = ld_frag(r.a[m], k, K);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if constexpr (MX) f.b[n][st] = ld_frag_mx((const uint8_t*)r.b[n], r.bs[n], k, K);
      else f.b[n][st] = ld_frag((const bf16_t*)r.b[n], k, K);
    }
  }
}

// acc[m][n] over this wave's share of K, then a fixed-order reduction over
// the four waves into red (LDS, 4 x 32 x 64 floats).
template <bool MX>
__device__ void sk_mainloop(const SkRows& r, int K, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  f32x4 acc[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nchunk = (int)ceil_div(K, 64);
  const int c0 = (wv * nchunk) / 4, c1 = ((wv + 1) * nchunk) / 4;
  if (c0 < c1) {
    SkFrag cur, nxt;
    sk_load<MX>(r, c0 * 64, K, cur);
    for (int c = c0; c < c1; ++c) {
      if (c + 1 < c1) sk_load<MX>(r, (c + 1) * 64, K, nxt);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 4; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[m][st], cur.b[n][st],
                                                                acc[m][n], 0, 0, 0);
      cur = nxt;
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[(wv * 32 + m * 16 + n * 4 + q) * 64 + lane] = acc[m][n][q];
  __syncthreads();
}

// Sum of value i (= m*16 + n*4 + q) of `lane` over the four waves, in order.
__device__ __forceinline__ float sk_sum(const float* red, int i, int lane) {
  float s = red[(0 * 32 + i) * 64 + lane];
  s += red[(1 * 32 + i) * 64 + lane];
  s += red[(2 * 32 + i) * 64 + lane];
  s += red[(3 * 32 + i) * 64 + lane];
  return s;
}

// Output position of value (m, n, q) of `lane`: tile row m*16 + 4*(lane/16) + q,
// tile column n*16 + lane%16 (the 16x16 accumulator layout).
template <bool MX>
__global__ __launch_bounds__(256) void skinny_glu_kernel(GroupedGluArgs a) {
  __shared__ float red[4 * 32 * 64];
  const int tile = blockIdx.y;
  if (tile >= a.tile_off[a.E]) return;
  const int e = expert_of_tile(a.tile_off, a.E, tile);
  const int row_lo = a.offsets[e] + (tile - a.tile_off[e]) * SK_BM;
  const int row_hi = min(min(a.offsets[e + 1], row_lo + SK_BM), a.rows_cap);
  const int f0 = blockIdx.x * 32;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15;

  SkRows r;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int row = row_lo + m * 16 + l16;
    const bf16_t* p = nullptr;
    if (row >= 0 && row < row_hi) {
      const int src = a.perm_src[row];
      const int t = src / a.topk;
      if (src >= 0 && t < a.T) p = (const bf16_t*)a.Z + (int64_t)t * a.ldz;
    }
    r.a[m] = p;
  }
  const int64_t wrow = (int64_t)e * a.F;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int f = f0 + (n & 1) * 16 + l16;
    const WOperand& w = (n < 2) ? a.Wg : a.Wv;
    const bool ok = f < a.F;
    if constexpr (MX) {
      r.b[n] = ok ? (const void*)((const uint8_t*)w.data + (wrow + f) * (a.K / 2)) : nullptr;
      r.bs[n] = ok ? w.scale + (wrow + f) * (a.K / 32) : nullptr;
    } else {
      r.b[n] = ok ? (const void*)((const bf16_t*)w.data + (wrow + f) * a.K) : nullptr;
      r.bs[n] = nullptr;
    }
  }
  sk_mainloop<MX>(r, a.K, red);

  const float inv_c = 1.0f / a.c;
  bf16_t* H = (bf16_t*)a.H;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pidx = wv * 4 + j;              // 16 (gate, up) pairs per lane
    const int m = pidx >> 3, n = (pidx >> 2) & 1, q = pidx & 3;
    const float g = sk_sum(red, m * 16 + n * 4 + q, lane);
    const float v = sk_sum(red, m * 16 + (n + 2) * 4 + q, lane);
    const int row = row_lo + m * 16 + 4 * (lane >> 4) + q;
    const int f = f0 + n * 16 + l16;
    if (row < row_hi && f < a.F) H[(int64_t)row * a.F + f] = f32_to_bf16(situ_glu(g, v, a.c, inv_c));
  }
}

template <bool MX>
__global__ __launch_bounds__(256) void skinny_down_kernel(GroupedDownArgs a) {
  __shared__ float red[4 * 32 * 64];
  const int tile = blockIdx.y;
  if (tile >= a.tile_off[a.E]) return;
  const int e = expert_of_tile(a.tile_off, a.E, tile);
  const int row_lo = a.offsets[e] + (tile - a.tile_off[e]) * SK_BM;
  const int row_hi = min(min(a.offsets[e + 1], row_lo + SK_BM), a.rows_cap);
  const int n0 = blockIdx.x * 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15;

  SkRows r;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int row = row_lo + m * 16 + l16;
    r.a[m] = (row >= 0 && row < row_hi) ? (const bf16_t*)a.H + (int64_t)row * a.ldh : nullptr;
  }
  const int64_t wrow = (int64_t)e * a.N;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int col = n0 + n * 16 + l16;
    const bool ok = col < a.N;
    if constexpr (MX) {
      r.b[n] = ok ? (const void*)((const uint8_t*)a.Wo.data + (wrow + col) * (a.K / 2)) : nullptr;
      r.bs[n] = ok ? a.Wo.scale + (wrow + col) * (a.K / 32) : nullptr;
    } else {
      r.b[n] = ok ? (const void*)((const bf16_t*)a.Wo.data + (wrow + col) * a.K) : nullptr;
      r.bs[n] = nullptr;
    }
  }
  sk_mainloop<MX>(r, a.K, red);

  bf16_t* O = (bf16_t*)a.O;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = wv * 8 + j;                 // 32 values per lane
    const int m = i >> 4, n = (i >> 2) & 3, q = i & 3;
    const float v = sk_sum(red, i, lane);
    const int row = row_lo + m * 16 + 4 * (lane >> 4) + q;
    const int col = n0 + n * 16 + l16;
    if (row < row_hi && col < a.N) O[(int64_t)row * a.N + col] = f32_to_bf16(v);
  }
}

// ---------------------------------------------------------------------------
// kernels (fp32 activations and weights): one thread per output
// ---------------------------------------------------------------------------

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

// The bf16 kernels use 72 KB of dynamic LDS (above the 64 KB default cap):
// raise the cap once per process for every instantiation.
int init_lds_caps() {
  static int status = -1;
  if (status >= 0) return status;
  const void* ks[] = {(const void*)dense_kernel<true>,        (const void*)dense_kernel<false>,
                      (const void*)glu_kernel<true>,          (const void*)glu_kernel<false>,
                      (const void*)grouped_glu_kernel<true>,  (const void*)grouped_glu_kernel<false>,
                      (const void*)grouped_down_kernel<true>, (const void*)grouped_down_kernel<false>,
                      (const void*)multiseg_kernel};
  status = 0;
  for (const void* k : ks) {
    hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) { status = (int)e; break; }
  }
  return status;
}

unsigned blocks_for(int64_t n) { return (unsigned)ceil_div(n, 256); }

}  // namespace

int grouped_bm(int act_dtype, int64_t rows, int E) {
  if (act_dtype == DT_F32) return 1;
  return rows <= (int64_t)SK_BM * E ? SK_BM : BM;
}

int launch_dense(const DenseArgs& a, hipStream_t stream) {
  if (a.M == 0) return 0;
  if (a.act_dtype != DT_F32) {
    if (int e = init_lds_caps()) return e;
  }
  if (a.act_dtype == DT_F32) {
    hipLaunchKernelGGL(dense_f32, dim3(blocks_for((int64_t)a.M * a.N)), dim3(256), 0, stream, a);
    return (int)hipGetLastError();
  }
  dim3 grid((unsigned)ceil_div(a.N, BN), (unsigned)ceil_div(a.M, BM));
  if (a.W.dtype == DT_MXFP4) {
    hipLaunchKernelGGL(dense_kernel<true>, grid, dim3(256), LDS_BYTES, stream, a);
  } else {
    hipLaunchKernelGGL(dense_kernel<false>, grid, dim3(256), LDS_BYTES, stream, a);
  }
  return (int)hipGetLastError();
}

int launch_glu(const GluArgs& a, hipStream_t stream) {
  if (a.M == 0) return 0;
  if (a.act_dtype != DT_F32) {
    if (int e = init_lds_caps()) return e;
  }
  if (a.act_dtype == DT_F32) {
    hipLaunchKernelGGL(glu_f32, dim3(blocks_for((int64_t)a.M * a.F)), dim3(256), 0, stream, a);
    return (int)hipGetLastError();
  }
  dim3 grid((unsigned)ceil_div(a.F, BN / 2), (unsigned)ceil_div(a.M, BM));
  if (a.Wg.dtype == DT_MXFP4) {
    hipLaunchKernelGGL(glu_kernel<true>, grid, dim3(256), LDS_BYTES, stream, a);
  } else {
    hipLaunchKernelGGL(glu_kernel<false>, grid, dim3(256), LDS_BYTES, stream, a);
  }
  return (int)hipGetLastError();
}

int launch_grouped_glu(const GroupedGluArgs& a, hipStream_t stream) {
  if (a.max_tiles == 0) return 0;
  if (a.act_dtype != DT_F32) {
    if (int e = init_lds_caps()) return e;
  }
  if (a.act_dtype == DT_F32) {
    // rows <= max_tiles when BM = 1 (the fp32 path uses one-row "tiles")
    hipLaunchKernelGGL(grouped_glu_f32, dim3(blocks_for((int64_t)a.max_tiles * a.F)), dim3(256), 0,
                       stream, a);
    return (int)hipGetLastError();
  }
  if (a.bm == SK_BM) {
    dim3 g((unsigned)ceil_div(a.F, 32), (unsigned)a.max_tiles);
    if (a.Wg.dtype == DT_MXFP4) hipLaunchKernelGGL(skinny_glu_kernel<true>, g, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(skinny_glu_kernel<false>, g, dim3(256), 0, stream, a);
    return (int)hipGetLastError();
  }
  if (a.bm != BM) return -1;
  dim3 grid((unsigned)ceil_div(a.F, BN / 2), (unsigned)a.max_tiles);
  if (a.Wg.dtype == DT_MXFP4) {
    hipLaunchKernelGGL(grouped_glu_kernel<true>, grid, dim3(256), LDS_BYTES, stream, a);
  } else {
    hipLaunchKernelGGL(grouped_glu_kernel<false>, grid, dim3(256), LDS_BYTES, stream, a);
  }
  return (int)hipGetLastError();
}

int launch_grouped_down(const GroupedDownArgs& a, hipStream_t stream) {
  if (a.max_tiles == 0) return 0;
  if (a.act_dtype != DT_F32) {
    if (int e = init_lds_caps()) return e;
  }
  if (a.act_dtype == DT_F32) {
    hipLaunchKernelGGL(grouped_down_f32, dim3(blocks_for((int64_t)a.max_tiles * a.N)), dim3(256), 0,
                       stream, a);
    return (int)hipGetLastError();
  }
  if (a.bm == SK_BM) {
    dim3 g((unsigned)ceil_div(a.N, 64), (unsigned)a.max_tiles);
    if (a.Wo.dtype == DT_MXFP4) hipLaunchKernelGGL(skinny_down_kernel<true>, g, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(skinny_down_kernel<false>, g, dim3(256), 0, stream, a);
    return (int)hipGetLastError();
  }
  if (a.bm != BM) return -1;
  dim3 grid((unsigned)ceil_div(a.N, BN), (unsigned)a.max_tiles);
  if (a.Wo.dtype == DT_MXFP4) {
    hipLaunchKernelGGL(grouped_down_kernel<true>, grid, dim3(256), LDS_BYTES, stream, a);
  } else {
    hipLaunchKernelGGL(grouped_down_kernel<false>, grid, dim3(256), LDS_BYTES, stream, a);
  }
  return (int)hipGetLastError();
}

int launch_multiseg(const MultiSegArgs& a, hipStream_t stream) {
  if (a.M == 0) return 0;
  if (a.act_dtype != DT_F32) {
    if (int e = init_lds_caps()) return e;
  }
  if (a.act_dtype == DT_F32) {
    hipLaunchKernelGGL(multiseg_f32, dim3(blocks_for((int64_t)a.M * a.N)), dim3(256), 0, stream, a);
    return (int)hipGetLastError();
  }
  dim3 grid((unsigned)ceil_div(a.N, BN), (unsigned)ceil_div(a.M, BM));
  hipLaunchKernelGGL(multiseg_kernel, grid, dim3(256), LDS_BYTES, stream, a);
  return (int)hipGetLastError();
}

}  // namespace moe
