// Matrix-core GEMMs of the Stable LatentMoE layer (gfx950, bf16 MFMA).
//
// Equations on "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか"
// (lilting.ch, section "K3のエキスパートは896個の小型LLMではない"):
//   z = W_down x                       -> dense_kernel      (latent down)
//   E_i(z) = W_o act(W_g z, W_v z)     -> grouped_glu_kernel + grouped_down_kernel
//   E_s(x), shared gate/up             -> glu_kernel
//   y = sum_s E_s(x) + W_up RMSNorm(u) -> multiseg_kernel: one GEMM whose K runs
//                                         over the shared experts' down projections
//                                         and then over W_up (a sum over experts
//                                         is a concatenation along K)
// Activation SiTU-GLU ("Kimi K3 テクニカルレポート", jiwasawa.github.io, section
// "幅のスケーリング: Stable LatentMoE"): act(g, v) = c tanh(SiLU(g)/c) c tanh(v/c),
// fused into the gate/up epilogue. MXFP4 weights ("Kimi K3 ... Open Frontier
// Intelligence", ai-tech-express.jp, section "MXFP4 Quantization-Aware
// Training") are decoded exactly to bf16 while they are staged into LDS, so
// the MFMA itself stays bf16.
//
// Engine: a block of WGM x WGN wave64s; each wave owns WM x WN tiles of
// v_mfma_f32_32x32x16_bf16 (fp32 accumulators). Dense GEMMs: 256 x 256 blocks
// of 8 waves (each 128 x 64) on the pipelined main loop. Grouped expert GEMMs: 128 x 256 blocks of 8
// waves (each 64 x 64, two waves per SIMD), since an expert's row count is
// rarely a multiple of 256; a wave whose rows are all padding skips its reads
// and MFMAs. bf16 operands go straight from global memory into LDS
// (buffer_load ... lds, 16 bytes per lane, no register staging) through a
// ring of NS stages of 64-k tiles (NS - 1 tiles in flight), into an unpadded
// layout of 128-byte rows whose 16-byte chunk c of row r sits in slot
// c ^ ((r >> 1) & 7): the MFMA operand reads (16 consecutive rows, same chunk,
// per LDS cycle) then hit distinct banks. Per K-tile a wave reads all its
// operand fragments into registers, then issues its MFMAs with the loads of a
// later tile spread between them (a load can stall the wave's issue while the
// address unit is busy; between MFMAs that time overlaps matrix work). MXFP4
// weights are loaded to registers, decoded, and written to the same layout
// (the dense GEMMs of large batches instead read a bf16 copy of their MXFP4
// weight, decoded once per call by decode_mxfp4_kernel).
// Loads are raw buffer loads from per-block bases: an offset past the buffer
// (rows past M, k past K, masked rows) returns zeros, so no load sits behind a
// branch. Every weight row is K-contiguous ([out, in] layout), so A and B
// tiles are both "rows x K" and stage the same way.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// WGM x WGN waves (NT = 64 WGM WGN threads); a wave owns WM x WN tiles of
// 32x32 MFMA, so the block tile is (32 WM WGM) x (32 WN WGN). K is staged BK
// (32 or 64) at a time through an NS-stage LDS ring (NS - 1 K-tiles in flight).
// CP: cache policy of the B (weight) loads, the buffer instructions' aux field
// (0, or kStream where each weight slice is read by one block only).
// Streaming loads: aux bit 1 of gfx950's buffer instructions sets `nt`, so the
// lines are not kept for reuse. Weights read once (one row tile per expert, at
// decode batch sizes) then stream at 6.7 TB/s instead of 6.3 (the K3 decode
// gate/up: 5.29 against 5.66-5.88 ms); where row tiles share a weight slice
// through L2 (prefill) it costs 3-5%.
constexpr int kStream = 2;

template <int WGM_, int WGN_, int WM_, int WN_, int BK_, int NS_, int CP_ = 0>
struct Cfg {
  static constexpr int WGM = WGM_, WGN = WGN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_, CP = CP_;
  static constexpr int NW = WGM * WGN, NT = 64 * NW;
  static constexpr int BM = 32 * WM * WGM, BN = 32 * WN * WGN;
  static constexpr int CH = BK / 8;            // 16-byte chunks per LDS row
  static constexpr int RPI = 64 / CH;          // tile rows per DMA instruction (1 KB)
  static constexpr int AR = BM / (NW * RPI);   // A: DMA loads per wave per stage
  static constexpr int BR = BN / (NW * RPI);   // B: DMA loads per wave per stage
  static constexpr int UR = BK / 32;           // MXFP4 32-element blocks per row per stage
  static constexpr int MXU = BN * UR / NT;     // MXFP4 (row, block) units per thread per stage
  static constexpr int STAGE = (BM + BN) * BK;   // bf16 elements per LDS stage
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(AR >= 1 && BR >= 1, "tile too small for the DMA pattern");
  static_assert(AR * NW * RPI == BM && BR * NW * RPI == BN, "DMA cover");
  static_assert(NS >= 2 && NS <= 5, "ring depth");
  // MXFP4 B (decoded through registers): whole (row, block) units per thread
  static constexpr bool MX_OK = MXU >= 1 && MXU * NT == BN * UR;
};
// Dense GEMMs (latent down, shared gate/up, output) at batch sizes that fill
// the chip: 256 x 256, 8 waves of 128 x 64, 2 stages of 64 KB, the pipelined
// main loop. bf16 weights only (MXFP4 ones are decoded to a bf16 copy first).
// On the K3 prefill shapes it runs the latent down in 0.79 ms and the shared
// experts (gate/up + output GEMM) in 4.26 ms, against 0.87 and 4.90 ms for
// 256 x 128 blocks of 4 waves with 3 stages of 48 KB (the same blocks on the
// pipelined loop: 0.88 and 5.01 ms; 320 x 256 blocks: 0.78 and 4.30 ms).
using DenseCfg = Cfg<2, 4, 4, 2, 64, 2>;
using GroupCfg = Cfg<2, 4, 2, 2, 64, 3, kStream>;   // 128 x 256, 8 waves, 3 stages of 48 KB
// Grouped expert GEMMs on bf16 weights with many rows per expert: 320 x 256,
// 8 waves of 160 x 64, the pipelined main loop (2 stages of 72 KB; 253 VGPRs).
#ifndef MOE_BIG_CFG
#define MOE_BIG_CFG Cfg<2, 4, 5, 2, 64, 2>
#endif
using GroupBigCfg = MOE_BIG_CFG;
using SplitCfg = Cfg<2, 2, 2, 2, 64, 3>;   // 128 x 128 (small batches, split K)

// ---------------------------------------------------------------------------
// operand staging
// ---------------------------------------------------------------------------

// bf16 rows by DMA: wave w fills tile rows w*RPI*N .. + RPI*N - 1 with one
// 1 KB buffer_load ... lds per q < N; lane i of load q takes tile row
// w*RPI*N + RPI*q + i/CH and writes LDS slot i%CH of it. The rows of load q
// come through resource r[sel[q]] (gate or up weights of a GLU tile; sel[q]
// is wave-uniform).
template <int N>
struct Rows {
  rsrc_t r[2];
  int sel[N];
  uint32_t off[N];  // byte offset of this lane's row of load q, or kOOB
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS layout of a tile row r (BK elements, CH chunks of 16 bytes): chunk c sits
// in slot c ^ swz(r). The MFMA operand reads take 16 consecutive rows at one
// chunk per LDS cycle; with the swizzle they cover all 64 banks.
//   BK = 64 (128-byte rows): rows r and r^1 differ in bank half and (r>>1)&7
//     takes 8 distinct values over the even (odd) rows of an aligned 16-row group.
//   BK = 32 (64-byte rows): rows r, r+4, r+8, r+12 share banks and (r>>2)&3
//     gives them 4 distinct slots.
template <class C>
__device__ __forceinline__ int swz(int r) {
  if constexpr (C::BK == 64) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// tile row of this lane's load q
template <class C, int N>
__device__ __forceinline__ int dma_row(int q) {
  return (threadIdx.x >> 6) * C::RPI * N + C::RPI * q + (threadIdx.x & 63) / C::CH;
}
// (wave row, wave column) of this thread in the WGM x WGN wave grid
template <class C>
__device__ __forceinline__ int wave_m() { return (threadIdx.x >> 6) / C::WGN; }
template <class C>
__device__ __forceinline__ int wave_n() { return (threadIdx.x >> 6) % C::WGN; }

template <class C, int N, int CP = 0>
__device__ __forceinline__ void dma_rows(const Rows<N>& rs, bf16_t* tile, int k0, int K) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: LDS base in M0
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const rsrc_t r = rs.sel[q] ? rs.r[1] : rs.r[0];
    const int row0 = wv * C::RPI * N + C::RPI * q;
    const int c = (lane % C::CH) ^ swz<C>(row0 + lane / C::CH);  // global chunk for this slot
    const int k = k0 + c * 8;
    const uint32_t o = rs.off[q];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(tile + row0 * C::BK), 16,
                                             (k < K && o != kOOB) ? o + 2u * (uint32_t)k : kOOB,
                                             0, 0, CP);
  }
}

// MXFP4 rows: unit j of thread t is tile row t / UR + (NT / UR) j and 32-element
// block t % UR of the stage.
template <int N>
struct MxRows {
  rsrc_t rp[2], rs[2];   // packed bytes, e8m0 scales (gate / up for the GLU tile)
  int sel[N];            // resource of unit j (wave-uniform)
  uint32_t poff[N];      // packed-row byte offset, or kOOB
  uint32_t soff[N];      // scale-row byte offset
};

struct MxStage {
  uint4 q;      // 32 e2m1 codes
  uint32_t s;   // e8m0 scale byte
};

template <class C>
__device__ __forceinline__ int mx_row(int j) { return threadIdx.x / C::UR + (C::NT / C::UR) * j; }

template <class C>
__device__ __forceinline__ void load_mx(const MxRows<C::MXU>& m, int k0, int K,
                                        MxStage (&st)[C::MXU]) {
  static_assert(C::MX_OK, "MXFP4 B needs whole (row, block) units per thread");
  const int k = k0 + (threadIdx.x % C::UR) * 32;
  const bool kin = k < K;
#pragma unroll
  for (int j = 0; j < C::MXU; ++j) {
    const bool ok = kin && m.poff[j] != kOOB;
    const rsrc_t rp = m.sel[j] ? m.rp[1] : m.rp[0];
    const rsrc_t rsc = m.sel[j] ? m.rs[1] : m.rs[0];
    st[j].q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rp, ok ? m.poff[j] + (uint32_t)(k / 2) : kOOB, 0, C::CP));
    st[j].s = __builtin_amdgcn_raw_buffer_load_b8(rsc, ok ? m.soff[j] + (uint32_t)(k / 32) : kOOB, 0, C::CP);
  }
}

// Decode of one 32-element MXFP4 block: gfx950's v_cvt_scalef32_pk_bf16_fp4
// turns the two e2m1 codes of one byte (low nibble first) into two bf16 scaled
// by an fp32 factor; with the factor 2^(s-127) of the e8m0 byte s the result is
// exact (a power-of-two scaling of a 2-significant-bit value; checked bit for
// bit against the value table for every code and every finite scale byte).
// Scale byte 255 (NaN in e8m0) is not supported.
template <class C>
__device__ __forceinline__ void store_mx(bf16_t* tile, const MxStage (&st)[C::MXU]) {
  const int part = threadIdx.x % C::UR;
#pragma unroll
  for (int j = 0; j < C::MXU; ++j) {
    const int row = mx_row<C>(j);
    const float scale = st[j].s == 0u ? 0x1p-127f : __uint_as_float(st[j].s << 23);
    const uint32_t q[4] = {st[j].q.x, st[j].q.y, st[j].q.z, st[j].q.w};
    bf16_t* dst = tile + row * C::BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the byte selector of the conversion is an immediate
      const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], scale, 0));
      const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], scale, 1));
      const uint32_t w2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], scale, 2));
      const uint32_t w3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], scale, 3));
      *(uint4*)(dst + 8 * ((part * 4 + i) ^ swz<C>(row))) = make_uint4(w0, w1, w2, w3);
    }
  }
}

// ---------------------------------------------------------------------------
// the MFMA main loop
// ---------------------------------------------------------------------------

template <class C>
struct Acc {
  f32x16 c[C::WM][C::WN];
};

template <class C>
__device__ __forceinline__ void acc_zero(Acc<C>& acc) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.c[i][j][r] = 0.0f;
}

// s_waitcnt with only the vector-memory counter limited to n.
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier without __syncthreads()'s release fence (that fence waits
// for every outstanding load, which would empty the DMA ring each K-tile).
// LDS needs no fence: each wave waits for its own DMA before it arrives here.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The LDS ring: one static array per stage (the compiler tracks DMA writes per
// array, so reading stage J waits only for the loads that fill stage J).
#define MOE_LDS_RING(C)                                                   \
  __shared__ __align__(16) bf16_t lds0[(C::NS > 0) ? C::STAGE : 1];    \
  __shared__ __align__(16) bf16_t lds1[(C::NS > 1) ? C::STAGE : 1];    \
  __shared__ __align__(16) bf16_t lds2[(C::NS > 2) ? C::STAGE : 1];    \
  __shared__ __align__(16) bf16_t lds3[(C::NS > 3) ? C::STAGE : 1];    \
  __shared__ __align__(16) bf16_t lds4[(C::NS > 4) ? C::STAGE : 1]
#define MOE_RING lds0, lds1, lds2, lds3, lds4

// Issue the loads of K-tile kt into stage buffer buf. Every load is
// unconditional (past K it reads zeros), so each stage issues the same number.
template <class C, bool B_MX>
__device__ __forceinline__ void stage_issue(bf16_t* buf, const Rows<C::AR>& ar, const Rows<C::BR>& br,
                                            const MxRows<C::MXU>& bm, int kt, int K) {
  if constexpr (B_MX) {
    // MXFP4 B: register loads first (the decode waits only for these), then A's DMA
    MxStage mx[C::MXU];
    load_mx<C>(bm, kt * C::BK, K, mx);
    dma_rows<C>(ar, buf, kt * C::BK, K);
    store_mx<C>(buf + C::BM * C::BK, mx);
  } else {
    dma_rows<C>(ar, buf, kt * C::BK, K);
    dma_rows<C, C::BR, C::CP>(br, buf + C::BM * C::BK, kt * C::BK, K);
  }
}

// Operand fragments of a whole stage, in registers.
template <class C>
struct Frags {
  bf16x8 a[C::BK / 16][C::WM], b[C::BK / 16][C::WN];
};

// NV: A fragments of this wave that hold rows of the problem (the others are
// all padding: no reads, no MFMAs). NV = 0 reads nothing.
template <class C, int NV>
__device__ __forceinline__ void read_frags(const bf16_t* As, const bf16_t* Bs, Frags<C>& f) {
  if constexpr (NV > 0) {
    const int lane = threadIdx.x & 63, wm = wave_m<C>(), wn = wave_n<C>();
    const int lr = lane & 31, lh = lane >> 5;
    // fragment rows start at multiples of 32, so the swizzle of row base + lr is swz(lr)
    const bf16_t* Aw = As + (wm * (C::BM / C::WGM) + lr) * C::BK;
    const bf16_t* Bw = Bs + (wn * (C::BN / C::WGN) + lr) * C::BK;
    const int sw = swz<C>(lr);
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
      const int slot = 8 * ((2 * ks + lh) ^ sw);
#pragma unroll
      for (int i = 0; i < NV; ++i) f.a[ks][i] = *(const bf16x8*)(Aw + i * 32 * C::BK + slot);
#pragma unroll
      for (int j = 0; j < C::WN; ++j) f.b[ks][j] = *(const bf16x8*)(Bw + j * 32 * C::BK + slot);
    }
  }
}

template <class C, int NV>
__device__ __forceinline__ void mma_frags(const Frags<C>& f, Acc<C>& acc) {
#pragma unroll
  for (int ks = 0; ks < C::BK / 16; ++ks)
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < C::WN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks][i], f.b[ks][j], acc.c[i][j], 0, 0, 0);
}

// One K-tile: stage kt (in R) has landed once only the later stages' loads are
// outstanding; after the barrier every wave is done with W (read one tile ago),
// which receives K-tile kt + NS - 1. The wave issues its fragment reads first,
// then the MFMAs with the next stage's loads spread between them: a load
// instruction can hold the wave's issue for a long time when the address unit
// is busy, and placed between MFMAs that time overlaps matrix work instead of
// adding to it.
template <class C, bool B_MX, int NV>
__device__ __forceinline__ void ring_step(bf16_t* R, bf16_t* W, const Rows<C::AR>& ar,
                                          const Rows<C::BR>& br, const MxRows<C::MXU>& bm, int kt,
                                          int K, Acc<C>& acc) {
  constexpr int kLoads = B_MX ? C::AR : C::AR + C::BR;  // DMA loads per thread per stage
  static_assert(kLoads * (C::NS - 2) < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoads * (C::NS - 2)));
  wg_barrier();
  Frags<C> f;
  // (NS = 2: the single buffer in flight is W itself, written after this barrier)
  read_frags<C, NV>(R, R + C::BM * C::BK, f);
  stage_issue<C, B_MX>(W, ar, br, bm, kt + C::NS - 1, K);
  mma_frags<C, NV>(f, acc);
  constexpr int kReads = NV > 0 ? C::BK / 16 * (NV + C::WN) : 0;
  constexpr int kMfma = C::BK / 16 * NV * C::WN;
  constexpr int kVmem = B_MX ? C::AR + 2 * C::MXU : C::AR + C::BR;
  constexpr int kPer = kMfma / kVmem > 0 ? kMfma / kVmem : 1;  // MFMAs between two loads
  if constexpr (kMfma == 0) return;
  __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);      // the stage's fragment reads
#pragma unroll
  for (int q = 0; q < kVmem; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);      // kPer MFMAs
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         // one load
  }
  if constexpr (kMfma > kPer * kVmem)
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kPer * kVmem, 0);
}

// MXFP4 B through registers, three K-tiles ahead of its LDS stage (NS = 3):
// step kt stores the decoded B of tile kt + 2 (loaded three steps ago, in q)
// into the free stage W next to A's DMA, then reloads q with tile kt + 5.
template <class C, int NV>
__device__ __forceinline__ void ring_step_mx(bf16_t* R, bf16_t* W, const Rows<C::AR>& ar,
                                             const MxRows<C::MXU>& bm, int kt, int K, Acc<C>& acc,
                                             MxStage (&q)[C::MXU]) {
  static_assert(C::NS == 3, "MXFP4 ring");
  constexpr int kMx = 2 * C::MXU;   // packed + scale load per unit
  // A of tile kt has landed once only A of kt+1 and B of kt+3, kt+4 are outstanding
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::AR + 2 * kMx));
  wg_barrier();
  Frags<C> f;
  read_frags<C, NV>(R, R + C::BM * C::BK, f);
  dma_rows<C>(ar, W, (kt + 2) * C::BK, K);
  store_mx<C>(W + C::BM * C::BK, q);
  load_mx<C>(bm, (kt + 5) * C::BK, K, q);
  mma_frags<C, NV>(f, acc);
  constexpr int kReads = NV > 0 ? C::BK / 16 * (NV + C::WN) : 0;
  constexpr int kMfma = C::BK / 16 * NV * C::WN;
  constexpr int kVmem = C::AR + kMx;
  constexpr int kPer = kMfma / kVmem > 0 ? kMfma / kVmem : 1;
  if constexpr (kMfma == 0) return;
  __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
  for (int v = 0; v < kVmem; ++v) {
    __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  if constexpr (kMfma > kPer * kVmem)
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kPer * kVmem, 0);
}

template <class C, int NV>
__device__ __forceinline__ void mainloop_mx(bf16_t* s0, bf16_t* s1, bf16_t* s2, const Rows<C::AR>& ar,
                                            const MxRows<C::MXU>& bm, int K, Acc<C>& acc) {
  const int nk = (int)ceil_div(K, C::BK);
  MxStage t[C::MXU], q0[C::MXU], q1[C::MXU], q2[C::MXU];   // q_i: B of tiles = i (mod 3)
  load_mx<C>(bm, 0, K, t);
  dma_rows<C>(ar, s0, 0, K);
  store_mx<C>(s0 + C::BM * C::BK, t);
  load_mx<C>(bm, C::BK, K, t);
  dma_rows<C>(ar, s1, C::BK, K);
  store_mx<C>(s1 + C::BM * C::BK, t);
  load_mx<C>(bm, 2 * C::BK, K, q2);
  load_mx<C>(bm, 3 * C::BK, K, q0);
  load_mx<C>(bm, 4 * C::BK, K, q1);
  for (int kt = 0; kt < nk; kt += 3) {
    ring_step_mx<C, NV>(s0, s2, ar, bm, kt, K, acc, q2);
    ring_step_mx<C, NV>(s1, s0, ar, bm, kt + 1, K, acc, q0);
    ring_step_mx<C, NV>(s2, s1, ar, bm, kt + 2, K, acc, q1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();
}

// acc += A_tile B_tile^T over k in [0, K) through the NS-stage ring. The
// K-tile count is rounded up to a multiple of NS; the extra tiles read zeros.
// A rows: `ar` (bf16 DMA); B rows: `br` (bf16 DMA) or `bm` (MXFP4, decoded
// through registers).
template <class C, bool B_MX, int NV = C::WM>
__device__ __forceinline__ void mainloop(bf16_t* s0, bf16_t* s1, bf16_t* s2, bf16_t* s3, bf16_t* s4,
                                         const Rows<C::AR>& ar, const Rows<C::BR>& br,
                                         const MxRows<C::MXU>& bm, int K, Acc<C>& acc) {
  if constexpr (B_MX && C::NS == 3) {
    mainloop_mx<C, NV>(s0, s1, s2, ar, bm, K, acc);
  } else {
    const int nk = (int)ceil_div(K, C::BK);
    stage_issue<C, B_MX>(s0, ar, br, bm, 0, K);
    if constexpr (C::NS > 2) stage_issue<C, B_MX>(s1, ar, br, bm, 1, K);
    if constexpr (C::NS > 3) stage_issue<C, B_MX>(s2, ar, br, bm, 2, K);
    if constexpr (C::NS > 4) stage_issue<C, B_MX>(s3, ar, br, bm, 3, K);
    for (int kt = 0; kt < nk; kt += C::NS) {
      if constexpr (C::NS == 2) {
        ring_step<C, B_MX, NV>(s0, s1, ar, br, bm, kt, K, acc);
        ring_step<C, B_MX, NV>(s1, s0, ar, br, bm, kt + 1, K, acc);
      } else if constexpr (C::NS == 3) {
        ring_step<C, B_MX, NV>(s0, s2, ar, br, bm, kt, K, acc);
        ring_step<C, B_MX, NV>(s1, s0, ar, br, bm, kt + 1, K, acc);
        ring_step<C, B_MX, NV>(s2, s1, ar, br, bm, kt + 2, K, acc);
      } else if constexpr (C::NS == 4) {
        ring_step<C, B_MX, NV>(s0, s3, ar, br, bm, kt, K, acc);
        ring_step<C, B_MX, NV>(s1, s0, ar, br, bm, kt + 1, K, acc);
        ring_step<C, B_MX, NV>(s2, s1, ar, br, bm, kt + 2, K, acc);
        ring_step<C, B_MX, NV>(s3, s2, ar, br, bm, kt + 3, K, acc);
      } else {
        ring_step<C, B_MX, NV>(s0, s4, ar, br, bm, kt, K, acc);
        ring_step<C, B_MX, NV>(s1, s0, ar, br, bm, kt + 1, K, acc);
        ring_step<C, B_MX, NV>(s2, s1, ar, br, bm, kt + 2, K, acc);
        ring_step<C, B_MX, NV>(s3, s2, ar, br, bm, kt + 3, K, acc);
        ring_step<C, B_MX, NV>(s4, s3, ar, br, bm, kt + 4, K, acc);
      }
    }
    // drain the trailing (zero) loads before the buffers are reused
    __builtin_amdgcn_s_waitcnt(0);
    wg_barrier();
  }
}

// mainloop for a tile whose rows at or past `valid_rows` are padding: each wave
// runs only the A fragments that hold real rows (wave-uniform choice).
template <class C, bool B_MX>
__device__ __forceinline__ void mainloop_rows(bf16_t* s0, bf16_t* s1, bf16_t* s2, bf16_t* s3, bf16_t* s4,
                                              const Rows<C::AR>& ar, const Rows<C::BR>& br,
                                              const MxRows<C::MXU>& bm, int K, int valid_rows,
                                              Acc<C>& acc) {
  static_assert(C::WM <= 4, "fragment dispatch");
  const int first = wave_m<C>() * (C::BM / C::WGM);
  const int nv = __builtin_amdgcn_readfirstlane(max(0, min(C::WM, (valid_rows - first + 31) / 32)));
  if (nv >= C::WM) mainloop<C, B_MX, C::WM>(s0, s1, s2, s3, s4, ar, br, bm, K, acc);
  else if (nv == 0) mainloop<C, B_MX, 0>(s0, s1, s2, s3, s4, ar, br, bm, K, acc);
  else if constexpr (C::WM > 1) {
    if (nv == 1) mainloop<C, B_MX, 1>(s0, s1, s2, s3, s4, ar, br, bm, K, acc);
    else if constexpr (C::WM > 2) {
      if (nv == 2) mainloop<C, B_MX, 2>(s0, s1, s2, s3, s4, ar, br, bm, K, acc);
      else if constexpr (C::WM > 3) mainloop<C, B_MX, 3>(s0, s1, s2, s3, s4, ar, br, bm, K, acc);
    }
  }
}

// ---------------------------------------------------------------------------
// the pipelined main loop (grouped expert GEMMs)
// ---------------------------------------------------------------------------
//
// Large wave tiles (WM x WN = 5 x 2 fragments, 160 x 64 per wave) cut the LDS
// bytes read per MFMA to 7/10 of the 64 x 64 tiles' (7 fragment reads per 10
// MFMAs), and 320 x 256 block tiles cut the L2-to-LDS bytes per flop to 0.6
// of the 128 x 256 tiles'. Fragment reads run one k-step (16 k) ahead of the
// MFMAs in two register sets, so a wave's matrix work never waits for its
// own LDS reads; the one workgroup barrier of a K-tile sits before that
// tile's last k-step, where every wave has its last fragments of the tile in
// registers: after it the stage just consumed takes the DMA of the K-tile NS
// ahead, and the first fragments of the next tile are read while the last
// k-step's MFMAs run.

template <class C>
struct KFrag {
  bf16x8 a[C::WM], b[C::WN];
};

// Fragments of k-step ks (16 k) of a stage: A fragments 0 .. NV-1 of this wave
// (the others hold padding rows only) and every B fragment.
template <class C, int NV>
__device__ __forceinline__ void read_kstep(const bf16_t* S, int ks, KFrag<C>& f) {
  if constexpr (NV > 0) {
    const int lane = threadIdx.x & 63, wm = wave_m<C>(), wn = wave_n<C>();
    const int lr = lane & 31, lh = lane >> 5;
    const bf16_t* Aw = S + (wm * (C::BM / C::WGM) + lr) * C::BK;
    const bf16_t* Bw = S + C::BM * C::BK + (wn * (C::BN / C::WGN) + lr) * C::BK;
    const int slot = 8 * ((2 * ks + lh) ^ swz<C>(lr));
#pragma unroll
    for (int i = 0; i < NV; ++i) f.a[i] = *(const bf16x8*)(Aw + i * 32 * C::BK + slot);
#pragma unroll
    for (int j = 0; j < C::WN; ++j) f.b[j] = *(const bf16x8*)(Bw + j * 32 * C::BK + slot);
  }
}

template <class C, int NV>
__device__ __forceinline__ void mma_kstep(const KFrag<C>& f, Acc<C>& acc) {
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j)
      acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc.c[i][j], 0, 0, 0);
}

// s_waitcnt: LDS/scalar counter 0 and the vector-memory counter limited to n.
constexpr int waitcnt_lgkm0_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (7 << 4); }

// k-steps KSI .. KS-2 of a K-tile in stage R: each issues the fragment reads of
// the next k-step (into the other register set) between its MFMAs. Even
// k-steps compute from f0, odd ones from f1 (compile-time choice: a runtime
// pick between the two sets would put them in scratch memory).
template <class C, int NV, int KSI>
__device__ __forceinline__ void pipe_ksteps(const bf16_t* R, Acc<C>& acc, KFrag<C>& f0, KFrag<C>& f1) {
  constexpr int KS = C::BK / 16;
  if constexpr (KSI + 1 < KS) {
    constexpr int kReads = NV > 0 ? NV + C::WN : 0;    // fragment reads per k-step
    constexpr int kMfma = NV * C::WN;                  // MFMAs per k-step
    if constexpr (KSI % 2 == 0) {
      read_kstep<C, NV>(R, KSI + 1, f1);
      mma_kstep<C, NV>(f0, acc);
    } else {
      read_kstep<C, NV>(R, KSI + 1, f0);
      mma_kstep<C, NV>(f1, acc);
    }
    if constexpr (kMfma > 0) {
      // one read after each of the first kReads MFMAs
#pragma unroll
      for (int q = 0; q < (kReads < kMfma ? kReads : kMfma); ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if constexpr (kReads > kMfma) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kMfma, 0);
      if constexpr (kMfma > kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
    }
    pipe_ksteps<C, NV, KSI + 1>(R, acc, f0, f1);
  }
}

// One K-tile kt: its stage R has landed and every wave passed the barrier
// that says so; f0 holds its k-step 0. Nx is the stage of tile kt + 1.
template <class C, int NV>
__device__ __forceinline__ void pipe_step(bf16_t* R, const bf16_t* Nx, const Rows<C::AR>& ar,
                                          const Rows<C::BR>& br, int kt, int K, Acc<C>& acc,
                                          KFrag<C>& f0, KFrag<C>& f1) {
  static_assert((C::BK / 16) % 2 == 0, "k-steps alternate between the two fragment sets");
  constexpr int kLoads = C::AR + C::BR;                // DMA per thread per stage
  static_assert(kLoads * (C::NS - 1) < 64, "vmcnt range");
  constexpr int kReads = NV > 0 ? NV + C::WN : 0;
  constexpr int kMfma = NV * C::WN;
  pipe_ksteps<C, NV, 0>(R, acc, f0, f1);
  // last k-step: its fragments (f1) are read; tile kt + 1 must land, and every
  // wave must be done with R before R takes tile kt + NS
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0_vm(kLoads * (C::NS - 2)));
  wg_barrier();
  dma_rows<C>(ar, R, (kt + C::NS) * C::BK, K);
  dma_rows<C, C::BR, C::CP>(br, R + C::BM * C::BK, (kt + C::NS) * C::BK, K);
  read_kstep<C, NV>(Nx, 0, f0);
  mma_kstep<C, NV>(f1, acc);
  if constexpr (kMfma > 0) {
    constexpr int kPer = kMfma / kLoads > 0 ? kMfma / kLoads : 1;   // MFMAs between two DMA
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
    if constexpr (kMfma > kPer * kLoads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kPer * kLoads, 0);
  }
}

template <class C>
__device__ __forceinline__ void stage_dma(bf16_t* S, const Rows<C::AR>& ar, const Rows<C::BR>& br, int kt,
                                          int K) {
  dma_rows<C>(ar, S, kt * C::BK, K);
  dma_rows<C, C::BR, C::CP>(br, S + C::BM * C::BK, kt * C::BK, K);
}

// acc += A_tile B_tile^T over k in [0, K), bf16 A and B by DMA through the
// NS-stage ring (all NS stages filled up front; K-tiles past K read zeros).
template <class C, int NV>
__device__ __forceinline__ void mainloop_pipe(bf16_t* s0, bf16_t* s1, bf16_t* s2, bf16_t* s3, bf16_t*,
                                              const Rows<C::AR>& ar, const Rows<C::BR>& br, int K,
                                              Acc<C>& acc) {
  static_assert(C::NS >= 2 && C::NS <= 4, "pipelined ring depth");
  const int nk = (int)ceil_div(K, C::BK);
  stage_dma<C>(s0, ar, br, 0, K);
  stage_dma<C>(s1, ar, br, 1, K);
  if constexpr (C::NS > 2) stage_dma<C>(s2, ar, br, 2, K);
  if constexpr (C::NS > 3) stage_dma<C>(s3, ar, br, 3, K);
  constexpr int kLoads = C::AR + C::BR;
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoads * (C::NS - 1)));
  wg_barrier();
  KFrag<C> f0, f1;
  read_kstep<C, NV>(s0, 0, f0);
  for (int kt = 0; kt < nk; kt += C::NS) {
    // whole rounds of NS K-tiles (tiles past K are zeros): a loop with one
    // exit keeps one copy of the accumulators
    if constexpr (C::NS == 2) {
      pipe_step<C, NV>(s0, s1, ar, br, kt, K, acc, f0, f1);
      pipe_step<C, NV>(s1, s0, ar, br, kt + 1, K, acc, f0, f1);
    } else if constexpr (C::NS == 3) {
      pipe_step<C, NV>(s0, s1, ar, br, kt, K, acc, f0, f1);
      pipe_step<C, NV>(s1, s2, ar, br, kt + 1, K, acc, f0, f1);
      pipe_step<C, NV>(s2, s0, ar, br, kt + 2, K, acc, f0, f1);
    } else {
      pipe_step<C, NV>(s0, s1, ar, br, kt, K, acc, f0, f1);
      pipe_step<C, NV>(s1, s2, ar, br, kt + 1, K, acc, f0, f1);
      pipe_step<C, NV>(s2, s3, ar, br, kt + 2, K, acc, f0, f1);
      pipe_step<C, NV>(s3, s0, ar, br, kt + 3, K, acc, f0, f1);
    }
  }
  // drain the trailing (zero) loads before the LDS is reused or the block ends
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();
}

// mainloop_pipe with NV = the largest count <= nv of this wave's 32-row
// fragments that hold valid rows (one instantiation per count).
template <class C, int NV>
__device__ __forceinline__ void pipe_dispatch(int nv, bf16_t* s0, bf16_t* s1, bf16_t* s2, bf16_t* s3,
                                              bf16_t* s4, const Rows<C::AR>& ar, const Rows<C::BR>& br,
                                              int K, Acc<C>& acc) {
  if constexpr (NV == 0) {
    mainloop_pipe<C, 0>(s0, s1, s2, s3, s4, ar, br, K, acc);
  } else {
    if (nv >= NV) mainloop_pipe<C, NV>(s0, s1, s2, s3, s4, ar, br, K, acc);
    else pipe_dispatch<C, NV - 1>(nv, s0, s1, s2, s3, s4, ar, br, K, acc);
  }
}

// mainloop_pipe for a tile whose rows at or past `valid_rows` are padding.
template <class C>
__device__ __forceinline__ void mainloop_pipe_rows(bf16_t* s0, bf16_t* s1, bf16_t* s2, bf16_t* s3,
                                                   bf16_t* s4, const Rows<C::AR>& ar,
                                                   const Rows<C::BR>& br, int K, int valid_rows,
                                                   Acc<C>& acc) {
  const int first = wave_m<C>() * (C::BM / C::WGM);
  const int nv = __builtin_amdgcn_readfirstlane(max(0, min(C::WM, (valid_rows - first + 31) / 32)));
  pipe_dispatch<C, C::WM>(nv, s0, s1, s2, s3, s4, ar, br, K, acc);
}

// Element (i, j, r) of this lane's accumulators sits at tile row / column
//   row = wm*BM/WGM + i*32 + 8*(r/4) + 4*(lane/32) + r%4,  col = wn*BN/WGN + j*32 + lane%32.
template <class C>
__device__ __forceinline__ int acc_row(int i, int r) {
  const int lane = threadIdx.x & 63;
  return wave_m<C>() * (C::BM / C::WGM) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
template <class C>
__device__ __forceinline__ int acc_col(int j) {
  const int lane = threadIdx.x & 63;
  return wave_n<C>() * (C::BN / C::WGN) + j * 32 + (lane & 31);
}

// ---------------------------------------------------------------------------
// operand set-up helpers
// ---------------------------------------------------------------------------

// A rows m0 + tile_row of a row-major [M, lda] bf16 matrix (rows >= M read zeros).
template <class C, int N>
__device__ __forceinline__ Rows<N> a_rows_dense(const void* A, int64_t lda, int m0, int M) {
  Rows<N> rs;
  const int nrows = max(0, min(M - m0, C::NW * C::RPI * N));
  rs.r[0] = rs.r[1] = make_rsrc((const bf16_t*)A + (int64_t)m0 * lda, (int64_t)nrows * lda * 2);
#pragma unroll
  for (int q = 0; q < N; ++q) {
    rs.sel[q] = 0;
    const int r = dma_row<C, N>(q);
    rs.off[q] = r < nrows ? (uint32_t)((int64_t)r * lda * 2) : kOOB;
  }
  return rs;
}

// B rows n0 + tile_row of a [N, K] bf16 matrix.
template <class C>
__device__ __forceinline__ Rows<C::BR> b_rows_plain(const void* W, int K, int n0, int N) {
  return a_rows_dense<C, C::BR>(W, K, n0, N);
}

template <class C>
__device__ __forceinline__ MxRows<C::MXU> b_mx_plain(const WOperand& w, int64_t row_base, int K, int n0,
                                                     int N) {
  MxRows<C::MXU> m;
  const int nrows = max(0, min(N - n0, C::BN));
  const int64_t r0 = row_base + n0;
  m.rp[0] = m.rp[1] = make_rsrc((const uint8_t*)w.data + r0 * (K / 2), (int64_t)nrows * (K / 2));
  m.rs[0] = m.rs[1] = make_rsrc(w.scale + r0 * (K / 32), (int64_t)nrows * (K / 32));
#pragma unroll
  for (int j = 0; j < C::MXU; ++j) {
    const int row = mx_row<C>(j);
    m.sel[j] = 0;
    m.poff[j] = row < nrows ? (uint32_t)(row * (K / 2)) : kOOB;
    m.soff[j] = row < nrows ? (uint32_t)(row * (K / 32)) : kOOB;
  }
  return m;
}

// GLU B tile: wave column wn covers tile rows wn*BN/WGN .. + BN/WGN: first the
// gate rows f0 + wn*H + (0 .. H-1) of Wg, then the same rows of Wv, with
// H = BN/(2 WGN). The block produces BN/2 outputs f0 .. f0 + BN/2 - 1. Wave w
// DMAs tile rows w*BN/NW .. + BN/NW in loads of RPI rows; each load lies inside
// one gate or up half (H is a multiple of RPI), so its resource is wave-uniform.
template <class C>
__device__ __forceinline__ int glu_half_rows() { return C::BN / (2 * C::WGN); }

template <class C>
__device__ __forceinline__ Rows<C::BR> b_rows_glu(const WOperand& g, const WOperand& v,
                                                  int64_t row_base, int K, int f0, int F) {
  constexpr int H = C::BN / (2 * C::WGN);
  static_assert(H % C::RPI == 0, "each load's B rows must be all gate or all up");
  Rows<C::BR> rs;
  const int nf = max(0, min(F - f0, C::BN / 2));  // valid outputs of this block
  rs.r[0] = make_rsrc((const bf16_t*)g.data + (row_base + f0) * K, (int64_t)nf * K * 2);
  rs.r[1] = make_rsrc((const bf16_t*)v.data + (row_base + f0) * K, (int64_t)nf * K * 2);
  const int wv = threadIdx.x >> 6;
  const int tr0 = wv * (C::BN / C::NW);                      // this wave's first tile row
#pragma unroll
  for (int q = 0; q < C::BR; ++q) {
    rs.sel[q] = __builtin_amdgcn_readfirstlane(((tr0 + C::RPI * q) % (2 * H)) >= H ? 1 : 0);
    const int tr = tr0 + C::RPI * q + (threadIdx.x & 63) / C::CH;
    const int fl = (tr / (2 * H)) * H + (tr % H);
    rs.off[q] = fl < nf ? (uint32_t)((int64_t)fl * K * 2) : kOOB;
  }
  return rs;
}

template <class C>
__device__ __forceinline__ MxRows<C::MXU> b_mx_glu(const WOperand& g, const WOperand& v,
                                                   int64_t row_base, int K, int f0, int F) {
  constexpr int H = C::BN / (2 * C::WGN);
  // a wave's units cover 64 / UR consecutive tile rows: all gate or all up
  static_assert(H % (64 / C::UR) == 0, "gate/up split must be wave-uniform");
  MxRows<C::MXU> m;
  const int nf = max(0, min(F - f0, C::BN / 2));
  m.rp[0] = make_rsrc((const uint8_t*)g.data + (row_base + f0) * (K / 2), (int64_t)nf * (K / 2));
  m.rs[0] = make_rsrc(g.scale + (row_base + f0) * (K / 32), (int64_t)nf * (K / 32));
  m.rp[1] = make_rsrc((const uint8_t*)v.data + (row_base + f0) * (K / 2), (int64_t)nf * (K / 2));
  m.rs[1] = make_rsrc(v.scale + (row_base + f0) * (K / 32), (int64_t)nf * (K / 32));
#pragma unroll
  for (int j = 0; j < C::MXU; ++j) {
    const int tr = mx_row<C>(j);                            // tile row
    m.sel[j] = __builtin_amdgcn_readfirstlane((tr % (2 * H)) >= H ? 1 : 0);
    const int fl = (tr / (2 * H)) * H + (tr % H);
    m.poff[j] = fl < nf ? (uint32_t)(fl * (K / 2)) : kOOB;
    m.soff[j] = fl < nf ? (uint32_t)(fl * (K / 32)) : kOOB;
  }
  return m;
}

// ---------------------------------------------------------------------------
// epilogues
// ---------------------------------------------------------------------------

// The epilogues store four consecutive bf16 of one row per lane (one 8-byte
// store) instead of one element: in the accumulator layout lane 4m + j of a
// 32 x 32 fragment holds column 4m + j of four consecutive rows per register
// group q, so a 4 x 4 transpose inside each quad of lanes (two DPP exchanges)
// gives lane 4m + j row j of columns 4m .. 4m + 3. Four times fewer store
// instructions; at K3 prefill sizes the element stores cost the expert down
// GEMM about 0.65 ms.
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {   // quad_perm [1, 0, 3, 2]
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {   // quad_perm [2, 3, 0, 1]
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}

// 4 x 4 transpose of bf16 inside each quad of lanes (every lane active). On
// entry lane 4m + j holds column j of the quad's block, rows p = 0..3 in e[p];
// on exit it holds row j, columns 0..3, as two dwords (lowest column first).
__device__ __forceinline__ uint2 quad_transpose(const bf16_t (&e)[4]) {
  const int j = threadIdx.x & 3;
  const bool odd = j & 1, hi = j & 2;
  // with lane j ^ 1: keep the two rows of j's parity, trade the other two
  const uint32_t ev = (uint32_t)e[0] | ((uint32_t)e[2] << 16);   // rows 0, 2
  const uint32_t od = (uint32_t)e[1] | ((uint32_t)e[3] << 16);   // rows 1, 3
  const uint32_t keep = odd ? od : ev;
  const uint32_t got = quad_xor1(odd ? ev : od);
  // rows (j & 1) and (j & 1) + 2 of columns (j & 2), (j & 2) + 1
  const uint32_t ra = odd ? (got & 0xFFFFu) | (keep << 16) : (keep & 0xFFFFu) | (got << 16);
  const uint32_t rb = odd ? (got >> 16) | (keep & 0xFFFF0000u) : (keep >> 16) | (got & 0xFFFF0000u);
  // with lane j ^ 2: keep row j, trade the other row
  const uint32_t keep2 = hi ? rb : ra;
  const uint32_t got2 = quad_xor2(hi ? ra : rb);
  return hi ? make_uint2(got2, keep2) : make_uint2(keep2, got2);
}

// bf16 columns n .. n + 3 of a row: one 8-byte store when all four are below
// N and the row stride keeps it aligned, else element by element.
__device__ __forceinline__ void store4(bf16_t* row, int n, int N, bool packed, uint2 v) {
  if (packed && n + 4 <= N) {
    *(uint2*)(row + n) = v;
  } else {
    const uint32_t w[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (n + c < N) row[n + c] = (bf16_t)w[c];
  }
}

// This lane's tile row / column after the quad transpose, for fragment row
// 32 i + 8 q and fragment column 32 j (add those).
template <class C>
__device__ __forceinline__ int quad_row() {
  const int lane = threadIdx.x & 63;
  return wave_m<C>() * (C::BM / C::WGM) + 4 * (lane >> 5) + (lane & 3);
}
__device__ __forceinline__ int quad_col() { return 4 * ((threadIdx.x & 31) >> 2); }

template <class C>
__device__ __forceinline__ void store_tile(const Acc<C>& acc, bf16_t* Cm, int64_t ldc, int m0, int n0,
                                           int M, int N) {
  const int r0 = m0 + quad_row<C>();
  const int c0 = n0 + wave_n<C>() * (C::BN / C::WGN) + quad_col();
  const bool packed = (ldc & 3) == 0;
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = r0 + 32 * i + 8 * q;
      if (__ballot(m < M) == 0) continue;      // no row of the group in range (wave-uniform)
#pragma unroll
      for (int j = 0; j < C::WN; ++j) {
        bf16_t e[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) e[p] = f32_to_bf16(acc.c[i][j][4 * q + p]);
        const uint2 v = quad_transpose(e);
        if (m < M) store4(Cm + (int64_t)m * ldc, c0 + 32 * j, N, packed, v);
      }
    }
}

// out_row(tile_row) -> output row index, or < 0 to skip
template <class C, typename RowMap>
__device__ __forceinline__ void store_glu(const Acc<C>& acc, bf16_t* H, int64_t ldh, int f0, int F,
                                          float c, RowMap out_row) {
  const float inv_c = 1.0f / c;
  const int r0 = quad_row<C>();
  const int c0 = f0 + wave_n<C>() * glu_half_rows<C>() + quad_col();
  const bool packed = (ldh & 3) == 0;
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t orow = out_row(r0 + 32 * i + 8 * q);
      if (__ballot(orow >= 0) == 0) continue;  // padding rows only (wave-uniform)
#pragma unroll
      for (int j = 0; j < C::WN / 2; ++j) {
        bf16_t e[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
          e[p] = f32_to_bf16(situ_glu(acc.c[i][j][4 * q + p], acc.c[i][j + C::WN / 2][4 * q + p], c, inv_c));
        const uint2 v = quad_transpose(e);
        if (orow >= 0) store4(H + orow * ldh, c0 + 32 * j, F, packed, v);
      }
    }
}

// XCD-aware block order. Workgroups are handed to the 8 XCDs round-robin
// (hardware id h runs on XCD h % 8), and each XCD has its own L2. Logical work
// item L = (h % 8) * chunk + h / 8, chunk = ceil(live / 8), gives every XCD one
// contiguous slice of the logical order, so blocks that share operands (the
// n-tiles of one row tile, the row tiles of one expert) run on the same XCD and
// share its L2. The 1-D grid holds at least 8 * ceil(live_max / 8) blocks;
// returns false for a block with nothing to do. (The mapping is a bijection
// onto [0, live) whatever the dispatch order; only the speed depends on it.)
constexpr int64_t xcd_grid(int64_t live_max) { return (live_max + 7) / 8 * 8; }

__device__ __forceinline__ bool xcd_item(int64_t live, int64_t& L) {
  const int64_t h = blockIdx.x;
  const int64_t chunk = (live + 7) / 8;
  const int64_t slot = h / 8;
  if (slot >= chunk) return false;
  L = (h % 8) * chunk + slot;
  return L < live;
}

// Tile order of a dense GEMM with mtn x ntn tiles: groups of kGroupM row
// tiles, and inside a group n-tile major, so the blocks that run together on
// one XCD (a contiguous run of work items) share a few A row tiles and a few B
// column tiles instead of one A tile and many B tiles: both stay in that XCD's
// L2 while the blocks walk K side by side.
// (The output GEMM, whose K runs over several segments, keeps row-major order:
// GM = 1.)
template <int GM>
__device__ __forceinline__ void dense_tile(int64_t L, int mtn, int ntn, int& mt, int& nt) {
  const int64_t per = (int64_t)GM * ntn;
  const int g = (int)(L / per);
  const int rows = min(GM, mtn - g * GM);   // row tiles in this group
  const int r = (int)(L - (int64_t)g * per);
  nt = r / rows;
  mt = g * GM + r % rows;
}
constexpr int kGroupM = 8;

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(DenseCfg::NT) void dense_kernel(DenseArgs a) {
  using C = DenseCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.N, C::BN);
  int64_t L;
  if (!xcd_item(ceil_div(a.M, C::BM) * ntn, L)) return;
  int mt, nt;
  dense_tile<kGroupM>(L, (int)ceil_div(a.M, C::BM), ntn, mt, nt);
  const int m0 = mt * C::BM, n0 = nt * C::BN;
  const Rows<C::AR> ar = a_rows_dense<C, C::AR>(a.A, a.lda, m0, a.M);
  Acc<C> acc;
  acc_zero(acc);
  const Rows<C::BR> br = b_rows_plain<C>(a.W.data, a.K, n0, a.N);
  mainloop_pipe<C, C::WM>(MOE_RING, ar, br, a.K, acc);
  store_tile(acc, (bf16_t*)a.C, a.ldc, m0, n0, a.M, a.N);
}

__global__ __launch_bounds__(DenseCfg::NT) void glu_kernel(GluArgs a) {
  using C = DenseCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.F, C::BN / 2);
  int64_t L;
  if (!xcd_item(ceil_div(a.M, C::BM) * ntn, L)) return;
  int mt, nt;
  dense_tile<kGroupM>(L, (int)ceil_div(a.M, C::BM), ntn, mt, nt);
  const int m0 = mt * C::BM, f0 = nt * (C::BN / 2);
  const Rows<C::AR> ar = a_rows_dense<C, C::AR>(a.A, a.lda, m0, a.M);
  Acc<C> acc;
  acc_zero(acc);
  const Rows<C::BR> br = b_rows_glu<C>(a.Wg, a.Wv, 0, a.K, f0, a.F);
  mainloop_pipe<C, C::WM>(MOE_RING, ar, br, a.K, acc);
  const int M = a.M;
  store_glu(acc, (bf16_t*)a.H, a.ldh, f0, a.F, a.c,
            [=](int tr) -> int64_t { return m0 + tr < M ? (int64_t)(m0 + tr) : -1; });
}

// Work item L of a grouped GEMM -> expert e, n-tile nt and row range
// [row_lo, row_hi). Logical order: expert by expert; inside an expert, n-tile
// major and row tile minor, so the row tiles that share one weight slice run
// side by side and read it through L2 once. Expert e owns items
// [tile_off[e], tile_off[e+1]) * ntn, so item L lies in the expert of tile
// L / ntn, whose tile_info entry {e, tile_off[e], count_e, offsets[e]} is the
// only table read. The values are the same for every lane: readfirstlane makes
// that visible to the compiler, so addresses built from them stay scalar
// (otherwise every buffer load would be wrapped in a waterfall loop).
template <int BM_>
__device__ __forceinline__ void grouped_item(const int32_t* tile_info, int ntn, int rows_cap, int64_t L,
                                             int& e, int& nt, int& row_lo, int& row_hi) {
  const int32_t* ti = tile_info + 4 * (L / ntn);
  e = __builtin_amdgcn_readfirstlane(ti[0]);
  const int t0 = __builtin_amdgcn_readfirstlane(ti[1]);
  const int cnt = __builtin_amdgcn_readfirstlane(ti[2]);
  const int r0 = __builtin_amdgcn_readfirstlane(ti[3]);
  const int mt = (cnt + BM_ - 1) / BM_;
  const int64_t local = L - (int64_t)t0 * ntn;
  nt = (int)(local / mt);
  row_lo = r0 + (int)(local % mt) * BM_;
  row_hi = min(min(r0 + cnt, row_lo + BM_), rows_cap);
}

template <bool B_MX>
__global__ __launch_bounds__(GroupCfg::NT) void grouped_glu_kernel(GroupedGluArgs a) {
  using C = GroupCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.F, C::BN / 2);
  int64_t L;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, L)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<C::BM>(a.tile_info, ntn, a.rows_cap, L, e, nt, row_lo, row_hi);
  const int f0 = nt * (C::BN / 2);
  // A: z rows of the tile's (token, slot) pairs, gathered through perm_src
  Rows<C::AR> ar;
  ar.r[0] = ar.r[1] = make_rsrc(a.Z, (int64_t)a.T * a.ldz * 2);
#pragma unroll
  for (int q = 0; q < C::AR; ++q) {
    ar.sel[q] = 0;
    const int row = row_lo + dma_row<C, C::AR>(q);
    uint32_t off = kOOB;
    if (row >= 0 && row < row_hi) {
      const int src = a.perm_src[row];
      const int t = src / a.topk;
      if (src >= 0 && t < a.T) off = (uint32_t)((int64_t)t * a.ldz * 2);
    }
    ar.off[q] = off;
  }
  const int64_t wrow = (int64_t)e * a.F;
  Acc<C> acc;
  acc_zero(acc);
  Rows<C::BR> br{};
  MxRows<C::MXU> bm{};
  if constexpr (B_MX) bm = b_mx_glu<C>(a.Wg, a.Wv, wrow, a.K, f0, a.F);
  else br = b_rows_glu<C>(a.Wg, a.Wv, wrow, a.K, f0, a.F);
  mainloop_rows<C, B_MX>(MOE_RING, ar, br, bm, a.K, row_hi - row_lo, acc);
  store_glu(acc, (bf16_t*)a.H, a.F, f0, a.F, a.c, [=](int tr) -> int64_t {
    const int r = row_lo + tr;
    return (r >= 0 && r < row_hi) ? (int64_t)r : -1;
  });
}

// grouped_glu_kernel<false> on GroupBigCfg tiles with the pipelined main loop
__global__ __launch_bounds__(GroupBigCfg::NT) void grouped_glu_big_kernel(GroupedGluArgs a) {
  using C = GroupBigCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.F, C::BN / 2);
  int64_t L;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, L)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<C::BM>(a.tile_info, ntn, a.rows_cap, L, e, nt, row_lo, row_hi);
  const int f0 = nt * (C::BN / 2);
  Rows<C::AR> ar;
  ar.r[0] = ar.r[1] = make_rsrc(a.Z, (int64_t)a.T * a.ldz * 2);
#pragma unroll
  for (int q = 0; q < C::AR; ++q) {
    ar.sel[q] = 0;
    const int row = row_lo + dma_row<C, C::AR>(q);
    uint32_t off = kOOB;
    if (row >= 0 && row < row_hi) {
      const int src = a.perm_src[row];
      const int t = src / a.topk;
      if (src >= 0 && t < a.T) off = (uint32_t)((int64_t)t * a.ldz * 2);
    }
    ar.off[q] = off;
  }
  const Rows<C::BR> br = b_rows_glu<C>(a.Wg, a.Wv, (int64_t)e * a.F, a.K, f0, a.F);
  Acc<C> acc;
  acc_zero(acc);
  mainloop_pipe_rows<C>(MOE_RING, ar, br, a.K, row_hi - row_lo, acc);
  store_glu(acc, (bf16_t*)a.H, a.F, f0, a.F, a.c, [=](int tr) -> int64_t {
    const int r = row_lo + tr;
    return (r >= 0 && r < row_hi) ? (int64_t)r : -1;
  });
}

__global__ __launch_bounds__(GroupBigCfg::NT) void grouped_down_big_kernel(GroupedDownArgs a) {
  using C = GroupBigCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.N, C::BN);
  int64_t L;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, L)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<C::BM>(a.tile_info, ntn, a.rows_cap, L, e, nt, row_lo, row_hi);
  const int n0 = nt * C::BN;
  const Rows<C::AR> ar = a_rows_dense<C, C::AR>(a.H, a.ldh, max(row_lo, 0), max(row_hi, 0));
  const Rows<C::BR> br = b_rows_plain<C>((const bf16_t*)a.Wo.data + (int64_t)e * a.N * a.K, a.K, n0, a.N);
  Acc<C> acc;
  acc_zero(acc);
  mainloop_pipe_rows<C>(MOE_RING, ar, br, a.K, row_hi - row_lo, acc);
  store_tile(acc, (bf16_t*)a.O, a.N, row_lo, n0, row_hi, a.N);
}

template <bool B_MX>
__global__ __launch_bounds__(GroupCfg::NT) void grouped_down_kernel(GroupedDownArgs a) {
  using C = GroupCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.N, C::BN);
  int64_t L;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, L)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<C::BM>(a.tile_info, ntn, a.rows_cap, L, e, nt, row_lo, row_hi);
  const int n0 = nt * C::BN;
  const Rows<C::AR> ar = a_rows_dense<C, C::AR>(a.H, a.ldh, max(row_lo, 0), max(row_hi, 0));
  const int64_t wrow = (int64_t)e * a.N;
  Acc<C> acc;
  acc_zero(acc);
  Rows<C::BR> br{};
  MxRows<C::MXU> bm{};
  if constexpr (B_MX) bm = b_mx_plain<C>(a.Wo, wrow, a.K, n0, a.N);
  else br = b_rows_plain<C>((const bf16_t*)a.Wo.data + wrow * a.K, a.K, n0, a.N);
  mainloop_rows<C, B_MX>(MOE_RING, ar, br, bm, a.K, row_hi - row_lo, acc);
  store_tile(acc, (bf16_t*)a.O, a.N, row_lo, n0, row_hi, a.N);
}

// Segments are visited in order, each through its own pass of the pipelined
// main loop into the same accumulators; every B is bf16.
__global__ __launch_bounds__(DenseCfg::NT) void multiseg_kernel(MultiSegArgs a) {
  using C = DenseCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.N, C::BN);
  int64_t L;
  if (!xcd_item(ceil_div(a.M, C::BM) * ntn, L)) return;
  int mt, nt;
  dense_tile<1>(L, (int)ceil_div(a.M, C::BM), ntn, mt, nt);
  const int m0 = mt * C::BM, n0 = nt * C::BN;
  Acc<C> acc;
  acc_zero(acc);
  for (int s = 0; s < a.nseg; ++s) {
    const Segment& sg = a.seg[s];
    const Rows<C::AR> ar = a_rows_dense<C, C::AR>(sg.A, sg.lda, m0, a.M);
    const Rows<C::BR> br = b_rows_plain<C>(sg.B.data, sg.K, n0, a.N);
    mainloop_pipe<C, C::WM>(MOE_RING, ar, br, sg.K, acc);
  }
  store_tile(acc, (bf16_t*)a.C, a.ldc, m0, n0, a.M, a.N);
}

// ---------------------------------------------------------------------------
// split-K path (few output rows: too few tiles to fill 256 CUs)
// ---------------------------------------------------------------------------


template <class C>
__device__ __forceinline__ void store_partial(const Acc<C>& acc, float* P, int64_t ldp, int m0, int n0,
                                              int M, int N) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      const int n = n0 + acc_col<C>(j);
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + acc_row<C>(i, r);
        if (m < M) P[(int64_t)m * ldp + n] = acc.c[i][j][r];
      }
    }
}

// GLU partial row: gate sums at [0, F), up sums at [F, 2F).
template <class C>
__device__ __forceinline__ void store_partial_glu(const Acc<C>& acc, float* P, int F, int f0, int m0,
                                                  int M) {
  const int lane = threadIdx.x & 63, wn = wave_n<C>();
#pragma unroll
  for (int j = 0; j < C::WN / 2; ++j) {
    const int f = f0 + wn * glu_half_rows<C>() + j * 32 + (lane & 31);
    if (f >= F) continue;
#pragma unroll
    for (int i = 0; i < C::WM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + acc_row<C>(i, r);
        if (m >= M) continue;
        float* row = P + (int64_t)m * 2 * F;
        row[f] = acc.c[i][j][r];
        row[F + f] = acc.c[i][j + C::WN / 2][r];
      }
  }
}

// Work item L -> (split, tile): split-major, so blocks that run together on
// one XCD read the same K range of A.
__device__ __forceinline__ void split_item(int64_t L, int64_t tiles, int ntn, int& sp, int& m0,
                                           int& n0, int BM, int BN) {
  sp = (int)(L / tiles);
  const int64_t tile = L % tiles;
  m0 = (int)(tile / ntn) * BM;
  n0 = (int)(tile % ntn) * BN;
}

// bf16 row operand shifted to column kb (row stride unchanged)
__device__ __forceinline__ WOperand shift_k(const WOperand& w, int kb) {
  if (w.dtype == DT_MXFP4) return WOperand{(const uint8_t*)w.data + kb / 2, w.scale + kb / 32, w.dtype};
  return WOperand{(const bf16_t*)w.data + kb, w.scale, w.dtype};
}

template <bool B_MX>
__global__ __launch_bounds__(SplitCfg::NT) void dense_split_kernel(DenseArgs a) {
  using C = SplitCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.N, C::BN);
  const int64_t tiles = ceil_div(a.M, C::BM) * ntn;
  int64_t L;
  if (!xcd_item(tiles * a.split.splits, L)) return;
  int sp, m0, n0;
  split_item(L, tiles, ntn, sp, m0, n0, C::BM, C::BN);
  const int kb = sp * a.split.kchunk, klen = min(a.K - kb, a.split.kchunk);
  const WOperand W = shift_k(a.W, kb);
  const Rows<C::AR> ar = a_rows_dense<C, C::AR>((const bf16_t*)a.A + kb, a.lda, m0, a.M);
  Rows<C::BR> br{};
  MxRows<C::MXU> bm{};
  if constexpr (B_MX) bm = b_mx_plain<C>(W, 0, a.K, n0, a.N);
  else br = b_rows_plain<C>(W.data, a.K, n0, a.N);
  Acc<C> acc;
  acc_zero(acc);
  mainloop<C, B_MX>(MOE_RING, ar, br, bm, klen, acc);
  store_partial(acc, a.P + (int64_t)sp * a.M * a.N, a.N, m0, n0, a.M, a.N);
}

__global__ __launch_bounds__(SplitCfg::NT) void glu_split_kernel(GluArgs a) {
  using C = SplitCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.F, C::BN / 2);
  const int64_t tiles = ceil_div(a.M, C::BM) * ntn;
  int64_t L;
  if (!xcd_item(tiles * a.split.splits, L)) return;
  int sp, m0, f0;
  split_item(L, tiles, ntn, sp, m0, f0, C::BM, C::BN / 2);
  const int kb = sp * a.split.kchunk, klen = min(a.K - kb, a.split.kchunk);
  const WOperand Wg = shift_k(a.Wg, kb), Wv = shift_k(a.Wv, kb);
  const Rows<C::AR> ar = a_rows_dense<C, C::AR>((const bf16_t*)a.A + kb, a.lda, m0, a.M);
  const Rows<C::BR> br = b_rows_glu<C>(Wg, Wv, 0, a.K, f0, a.F);
  Acc<C> acc;
  acc_zero(acc);
  mainloop<C, false>(MOE_RING, ar, br, MxRows<C::MXU>{}, klen, acc);
  store_partial_glu(acc, a.P + (int64_t)sp * a.M * 2 * a.F, a.F, f0, m0, a.M);
}

// One work item per (segment, tile); segment s writes partial slice s.
template <bool LAST_MX>
__global__ __launch_bounds__(SplitCfg::NT) void multiseg_split_kernel(MultiSegArgs a, int s0, int ns) {
  using C = SplitCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.N, C::BN);
  const int64_t tiles = ceil_div(a.M, C::BM) * ntn;
  int64_t L;
  if (!xcd_item(tiles * ns, L)) return;
  int s, m0, n0;
  split_item(L, tiles, ntn, s, m0, n0, C::BM, C::BN);
  s += s0;
  const Segment& sg = a.seg[s];
  const Rows<C::AR> ar = a_rows_dense<C, C::AR>(sg.A, sg.lda, m0, a.M);
  Acc<C> acc;
  acc_zero(acc);
  if (LAST_MX && s == a.nseg - 1) {
    const MxRows<C::MXU> bm = b_mx_plain<C>(sg.B, 0, sg.K, n0, a.N);
    mainloop<C, true>(MOE_RING, ar, Rows<C::BR>{}, bm, sg.K, acc);
  } else {
    const Rows<C::BR> br = b_rows_plain<C>(sg.B.data, sg.K, n0, a.N);
    mainloop<C, false>(MOE_RING, ar, br, MxRows<C::MXU>{}, sg.K, acc);
  }
  store_partial(acc, a.P + (int64_t)s * a.M * a.N, a.N, m0, n0, a.M, a.N);
}

// C[m, n] = bf16(sum over slices in ascending order); 4 columns per thread.
__global__ __launch_bounds__(256) void reduce_store_kernel(const float* __restrict__ P, int slices,
                                                           int M, int N, bf16_t* __restrict__ Cm,
                                                           int64_t ldc) {
  const int64_t stride = (int64_t)M * N, n4 = stride / 4;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4;
       q += (int64_t)gridDim.x * blockDim.x) {
    float4 v = ((const float4*)P)[q];
    for (int s = 1; s < slices; ++s) {
      const float4 w = ((const float4*)(P + s * stride))[q];
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    const int64_t e = q * 4, m = e / N, n = e % N;
    const uint32_t lo = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
    *(uint2*)(Cm + m * ldc + n) = make_uint2(lo, hi);
  }
}

// H[m, f] = bf16(act(sum gate, sum up)) from GLU partial rows [gate F | up F].
__global__ __launch_bounds__(256) void reduce_glu_kernel(const float* __restrict__ P, int slices, int M,
                                                         int F, float c, bf16_t* __restrict__ H,
                                                         int64_t ldh) {
  const int64_t stride = (int64_t)M * 2 * F, n4 = (int64_t)M * F / 4;
  const float inv_c = 1.0f / c;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = q * 4, m = e / F, f = e % F;
    const float* g0 = P + m * 2 * F + f;
    float4 g = *(const float4*)g0, u = *(const float4*)(g0 + F);
    for (int s = 1; s < slices; ++s) {
      const float4 wg = *(const float4*)(g0 + s * stride), wu = *(const float4*)(g0 + s * stride + F);
      g.x += wg.x; g.y += wg.y; g.z += wg.z; g.w += wg.w;
      u.x += wu.x; u.y += wu.y; u.z += wu.z; u.w += wu.w;
    }
    const uint32_t lo = (uint32_t)f32_to_bf16(situ_glu(g.x, u.x, c, inv_c)) |
                        ((uint32_t)f32_to_bf16(situ_glu(g.y, u.y, c, inv_c)) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(situ_glu(g.z, u.z, c, inv_c)) |
                        ((uint32_t)f32_to_bf16(situ_glu(g.w, u.w, c, inv_c)) << 16);
    *(uint2*)(H + m * ldh + f) = make_uint2(lo, hi);
  }
}

int reduce_blocks(int64_t n4) { return (int)(ceil_div(n4, 256) < 2048 ? ceil_div(n4, 256) : 2048); }

// Approximate router logits (the exact routing is decided in router.hip):
// 128 x 128 tiles of x W_r^T, K split over `splits` blocks whose fp32 partial
// sums are added atomically (their order does not matter: the logits only
// bound the fixed-order ones). Two 32 KB stages, so that two blocks share a CU:
// at the K3 prefill batch (896 tiles of 112 K-tiles) that halves the kernel's
// time against three stages and one block per CU (0.50 against 0.93 ms).
#ifndef MOE_LOGIT_CFG
#define MOE_LOGIT_CFG Cfg<2, 2, 2, 2, 64, 2>
#endif
using LogitCfg = MOE_LOGIT_CFG;

__global__ __launch_bounds__(LogitCfg::NT) void logits_kernel(LogitsArgs a) {
  using C = LogitCfg;
  MOE_LDS_RING(C);
  const int ntn = (int)ceil_div(a.E, C::BN), ntm = (int)ceil_div(a.T, C::BM);
  int64_t L;
  if (!xcd_item((int64_t)ntm * ntn * a.splits, L)) return;
  const int sp = (int)(L % a.splits);
  const int64_t rest = L / a.splits;
  const int m0 = (int)(rest / ntn) * C::BM, n0 = (int)(rest % ntn) * C::BN;
  const int kchunk = (int)ceil_div(ceil_div(a.d, a.splits), LogitCfg::BK) * LogitCfg::BK;
  const int k0 = sp * kchunk;
  const int klen = min(a.d - k0, kchunk);
  if (klen <= 0) return;
  const Rows<C::AR> ar = a_rows_dense<C, C::AR>((const bf16_t*)a.x + k0, a.d, m0, a.T);
  const Rows<C::BR> br = a_rows_dense<C, C::BR>((const bf16_t*)a.W + k0, a.d, n0, a.E);
  Acc<C> acc;
  acc_zero(acc);
  mainloop<C, false>(MOE_RING, ar, br, MxRows<C::MXU>{}, klen, acc);
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      const int n = n0 + acc_col<C>(j);
      if (n >= a.E) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + acc_row<C>(i, r);
        if (m >= a.T) continue;
        float* dst = a.L + (int64_t)m * a.E + n;
        if (a.splits == 1) *dst = acc.c[i][j][r];
        else atomicAdd(dst, acc.c[i][j][r]);
      }
    }
}

__global__ void zero_f32(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

// bf16 copy of a row-major MXFP4 weight (packed [rows, K/2], scales
// [rows, K/32]; K % 32 == 0): one thread per 32-element block, decoded with
// the conversion and scale rule of store_mx (exact), 64 bytes written.
__global__ __launch_bounds__(256) void decode_mxfp4_kernel(const uint8_t* __restrict__ packed,
                                                           const uint8_t* __restrict__ scale,
                                                           bf16_t* __restrict__ out, int64_t blocks) {
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < blocks;
       u += (int64_t)gridDim.x * blockDim.x) {
    const uint4 q4 = *(const uint4*)(packed + 16 * u);
    const uint32_t sb = scale[u];
    const float sc = sb == 0u ? 0x1p-127f : __uint_as_float(sb << 23);
    const uint32_t q[4] = {q4.x, q4.y, q4.z, q4.w};
    uint4* dst = (uint4*)(out + 32 * u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], sc, 0));
      const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], sc, 1));
      const uint32_t w2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], sc, 2));
      const uint32_t w3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], sc, 3));
      dst[i] = make_uint4(w0, w1, w2, w3);
    }
  }
}

// ---------------------------------------------------------------------------
// Scaled-MFMA expert GEMMs: MXFP8 activations x MXFP4 weights
// ---------------------------------------------------------------------------
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with A = E4M3 activation rows and B = E2M1
// weight rows, each with one e8m0 scale per 32 elements along K. Operand
// layout (lane l, h = l / 32; checked on the GPU against a host product for
// random codes and scales): A lane l holds row l % 32, bytes 0-15 at
// k = 16h .. 16h+15 and bytes 16-31 at k = 32 + 16h .. 32 + 16h + 15 of the
// instruction's 64; B lane l holds row l % 32, elements k = 32h .. 32h + 31
// (16 bytes, low nibble first); byte 0 of each lane's scale register is the
// scale of its row's k-block h. The accumulator layout is that of
// v_mfma_f32_32x32x16_bf16, so the bf16 engine's epilogues apply.
//
// Block 128 x kBN (8 waves in a 2 x 4 grid, each 64 x kBN/4), K staged 128
// elements at a time through a 3-stage LDS ring; per stage: A 128 rows x 128
// bytes, B kBN rows x 64 bytes (both swizzled as the bf16 layouts of the same
// row lengths), and per wave two 256-byte scale areas (the four scale bytes of
// the stage of its 16 A rows and its kBRW B rows). Wave w loads A rows
// 16w .. 16w+15 (2 DMA), B rows kBRW w .. kBRW w + kBRW - 1 (kBRW / 16 DMA)
// and their scales (2 DMA).
namespace mx8 {
#ifndef MOE_MX8_BN
#define MOE_MX8_BN 512
#endif
constexpr int kBN = MOE_MX8_BN;                // B rows (weights) per block: 256 or 512
constexpr int kBRW = kBN / 8;                  // B rows per wave's loads
constexpr int kBQ = kBRW / 16;                 // B DMA per wave per stage
constexpr int kBK = 128;                       // elements per stage
constexpr int kArow = kBK, kBrow = kBK / 2;    // bytes per row per stage
constexpr int kA = 128 * kArow, kB = kBN * kBrow, kS = 8 * 256;
constexpr int kStage = kA + kB + 2 * kS;       // bytes: A | B | A scales | B scales
constexpr int kNS = 3;
constexpr int kLoads = 2 + kBQ + 2;            // DMA per wave per stage
using L = Cfg<2, 4, 2, kBN / 128, 64, 3>;      // accumulator / epilogue layout (128 x kBN)
static_assert(L::BM == 128 && L::BN == kBN && L::NT == 512 && kBRW <= 64, "layout");

__device__ __forceinline__ int swz_a(int r) { return (r >> 1) & 7; }   // 128-byte rows
__device__ __forceinline__ int swz_b(int r) { return (r >> 2) & 3; }   // 64-byte rows

// Per-lane sources of one wave's stage loads: row byte offsets of the data
// loads (kOOB: none) and of the scale loads.
struct Src {
  rsrc_t ra, rb, rsa, rsb;      // A codes, B packed, A scales, B scales
  uint32_t aoff[2], boff[kBQ];  // data row offsets of this lane's rows in load q
  uint32_t asoff, bsoff;        // scale offsets of stage 0 (lanes 0-15 / 0 .. kBRW-1), or kOOB
  uint32_t bdstep, bsstep;      // B data / scale bytes between stages: 64 / 4 (row-major) or
                                // 128 / 256 (tiled layout)
};

// Stage kt into buf (LDS byte buffer). A chunk c (16 bytes) of tile row r sits
// in slot c ^ swz_a(r); B chunk c in slot c ^ swz_b(r). B chunk c of a row's
// stage kt is at its offset boff + bdstep kt + 16 c in either layout.
template <int CP>
__device__ __forceinline__ void stage_issue(uint8_t* buf, const Src& s, int kt, int K) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row0 = 16 * w + 8 * q;          // A: 8 rows of 8 chunks per load
    const int c = (lane & 7) ^ swz_a(row0 + (lane >> 3));
    const int k = kt * kBK + 16 * c;          // fp8: 16 elements per chunk
    const uint32_t o = s.aoff[q];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.ra, (lds_ptr_t)(buf + row0 * kArow), 16,
                                             (k < K && o != kOOB) ? o + (uint32_t)k : kOOB, 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < kBQ; ++q) {
    const int row0 = kBRW * w + 16 * q;       // B: 16 rows of 4 chunks per load
    const int c = (lane & 3) ^ swz_b(row0 + (lane >> 2));
    const int k = kt * kBK + 32 * c;          // fp4: 32 elements per chunk
    const uint32_t o = s.boff[q];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rb, (lds_ptr_t)(buf + kA + row0 * kBrow), 16,
                                             (k < K && o != kOOB) ? o + s.bdstep * (uint32_t)kt + 16u * (uint32_t)c
                                                                  : kOOB,
                                             0, 0, CP);
  }
  // four scale bytes (k-blocks 4kt .. 4kt+3) per row; K % 128 == 0
  const bool kin = kt * kBK < K;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rsa, (lds_ptr_t)(buf + kA + kB + 256 * w), 4,
                                           (kin && s.asoff != kOOB) ? s.asoff + 4u * (uint32_t)kt : kOOB,
                                           0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rsb, (lds_ptr_t)(buf + kA + kB + kS + 256 * w), 4,
                                           (kin && s.bsoff != kOOB) ? s.bsoff + s.bsstep * (uint32_t)kt : kOOB,
                                           0, 0, CP);
}

typedef int v8i __attribute__((ext_vector_type(8)));

struct Frags {
  v8i a[2][2];            // [k-step][A fragment]
  v8i b[2][L::WN];        // [k-step][B fragment] (first 16 bytes used)
  uint32_t sa[2], sb[L::WN];  // scale dwords (blocks 4kt .. 4kt+3) of this lane's rows
};

template <int NV>
__device__ __forceinline__ void read_frags(const uint8_t* buf, Frags& f) {
  if constexpr (NV > 0) {
    const int lane = threadIdx.x & 63, wm = wave_m<L>(), wn = wave_n<L>();
    const int lr = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int r = wm * 64 + i * 32 + lr;                 // A tile row
      const uint8_t* row = buf + r * kArow;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 lo = *(const uint4*)(row + 16 * ((4 * s + h) ^ swz_a(r)));
        const uint4 hi = *(const uint4*)(row + 16 * ((4 * s + 2 + h) ^ swz_a(r)));
        f.a[s][i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      f.sa[i] = *(const uint32_t*)(buf + kA + kB + 256 * (r >> 4) + 4 * (r & 15));
    }
#pragma unroll
    for (int j = 0; j < L::WN; ++j) {
      const int n = wn * (kBN / 4) + j * 32 + lr;          // B tile row
      const uint8_t* row = buf + kA + n * kBrow;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 v = *(const uint4*)(row + 16 * ((2 * s + h) ^ swz_b(n)));
        f.b[s][j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
      f.sb[j] = *(const uint32_t*)(buf + kA + kB + kS + 256 * (n / kBRW) + 4 * (n % kBRW));
    }
  }
}

template <int NV>
__device__ __forceinline__ void mma(const Frags& f, Acc<L>& acc) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < L::WN; ++j)
        // byte 0 of the scale operand: this lane's row, k-block 4kt + 2s + h
        acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.a[s][i], f.b[s][j], acc.c[i][j], 0, 4, 0, (int)(f.sa[i] >> (8 * (2 * s + h))), 0,
            (int)(f.sb[j] >> (8 * (2 * s + h))));
}

template <int NV, int CP>
__device__ __forceinline__ void ring_step(const uint8_t* R, uint8_t* W, const Src& s, int kt, int K,
                                          Acc<L>& acc) {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoads * (kNS - 2)));
  wg_barrier();
  Frags f;
  read_frags<NV>(R, f);
  stage_issue<CP>(W, s, kt + kNS - 1, K);
  mma<NV>(f, acc);
}

template <int NV, int CP>
__device__ __forceinline__ void mainloop(uint8_t* s0, uint8_t* s1, uint8_t* s2, const Src& s, int K,
                                         Acc<L>& acc) {
  const int nk = (int)ceil_div(K, kBK);
  stage_issue<CP>(s0, s, 0, K);
  stage_issue<CP>(s1, s, 1, K);
  for (int kt = 0; kt < nk; kt += 3) {
    ring_step<NV, CP>(s0, s2, s, kt, K, acc);
    ring_step<NV, CP>(s1, s0, s, kt + 1, K, acc);
    ring_step<NV, CP>(s2, s1, s, kt + 2, K, acc);
  }
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();
}

// CP: cache policy of the weight loads (kStream at decode batch sizes)
template <int CP>
__device__ __forceinline__ void mainloop_rows(uint8_t* s0, uint8_t* s1, uint8_t* s2, const Src& s, int K,
                                              int valid_rows, Acc<L>& acc) {
  const int first = wave_m<L>() * 64;
  const int nv = __builtin_amdgcn_readfirstlane(max(0, min(2, (valid_rows - first + 31) / 32)));
  if (nv >= 2) mainloop<2, CP>(s0, s1, s2, s, K, acc);
  else if (nv == 1) mainloop<1, CP>(s0, s1, s2, s, K, acc);
  else mainloop<0, CP>(s0, s1, s2, s, K, acc);
}

#define MOE_MX8_RING                                          \
  __shared__ __align__(16) uint8_t mx0[mx8::kStage];          \
  __shared__ __align__(16) uint8_t mx1[mx8::kStage];          \
  __shared__ __align__(16) uint8_t mx2[mx8::kStage]

// B offsets at stage 0 and the steps between stages. Row-major: packed row r
// at r K/2 (64 bytes a stage), scales at r K/32 (4 bytes a stage). Tiled
// layout: the packed bytes of rows 2p and 2p+1 interleaved per stage
// ([R/2][K/128][2][64]), so that a stage of a row pair is one 128-byte cache
// line; the scales stage-tiled ([R/64][K/128][64][4]), so that a stage's
// scales of 64 rows are 256 contiguous bytes instead of 4 bytes from each of
// 64 rows. Row r of the data load is relative to an even row; `first` (the
// wave's first scale row) is 64-aligned in absolute rows (the callers require
// d_ff, d_latent % 128).
__device__ __forceinline__ uint32_t b_data_off(bool tiled, int r, int K) {
  return tiled ? (uint32_t)((r >> 1) * K + (r & 1) * 64) : (uint32_t)(r * (K / 2));
}
__device__ __forceinline__ void b_scale_src(Src& s, bool tiled, int first, int lane, int K, bool live) {
  s.bdstep = tiled ? 128u : 64u;
  s.bsstep = tiled ? 256u : 4u;
  s.bsoff = !live ? kOOB
                  : tiled ? (uint32_t)(first * (K / 32) + 4 * lane) : (uint32_t)((first + lane) * (K / 32));
}

// B sources of a GLU tile (H = kBRW = the outputs of one consumer column):
// tile rows 2Hc .. 2Hc+H-1 are the gate rows of outputs f0 + Hc .. + H-1, rows
// 2Hc+H .. 2Hc+2H-1 their up rows; wave w's kBRW rows lie in one half (gate
// for even w, up for odd w).
__device__ __forceinline__ void b_src_glu(Src& s, const WOperand& g, const WOperand& v, int64_t row_base,
                                          int K, int f0, int F, bool tiled) {
  static_assert(kBN / (2 * 4) == kBRW, "a wave's B rows are one half of a consumer column");
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nf = max(0, min(F - f0, kBN / 2));
  const bool up = (w & 1) != 0;
  const WOperand& src = up ? v : g;
  s.rb = make_rsrc((const uint8_t*)src.data + (row_base + f0) * (K / 2), (int64_t)nf * (K / 2));
  s.rsb = make_rsrc(src.scale + (row_base + f0) * (K / 32), (int64_t)nf * (K / 32));
  const int fbase = (w >> 1) * kBRW;                     // output of this wave's first row
#pragma unroll
  for (int q = 0; q < kBQ; ++q) {
    const int fl = fbase + 16 * q + (lane >> 2);
    s.boff[q] = fl < nf ? b_data_off(tiled, fl, K) : kOOB;
  }
  b_scale_src(s, tiled, fbase, lane, K, lane < kBRW && fbase + lane < nf);
}

__device__ __forceinline__ void b_src_plain(Src& s, const WOperand& wo, int64_t row_base, int K, int n0,
                                            int N, bool tiled) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nrows = max(0, min(N - n0, kBN));
  s.rb = make_rsrc((const uint8_t*)wo.data + (row_base + n0) * (K / 2), (int64_t)nrows * (K / 2));
  s.rsb = make_rsrc(wo.scale + (row_base + n0) * (K / 32), (int64_t)nrows * (K / 32));
#pragma unroll
  for (int q = 0; q < kBQ; ++q) {
    const int r = kBRW * w + 16 * q + (lane >> 2);
    s.boff[q] = r < nrows ? b_data_off(tiled, r, K) : kOOB;
  }
  b_scale_src(s, tiled, kBRW * w, lane, K, lane < kBRW && kBRW * w + lane < nrows);
}
}  // namespace mx8

namespace mx8 {
// GLU epilogue that writes h already in MXFP8 (codes [rows, F], e8m0 scales
// [rows, F/32]), the down GEMM's input, instead of bf16 h for a separate
// quantisation pass: the same numbers as rounding h to bf16 and quantising
// that row by row, step for step as the standalone quantiser does. The tile's
// bf16 h (128 rows x 256 outputs) first goes to the LDS ring, free after the
// main loop (rows 0-63 in lo, 64-127 in hi, 512 bytes a row); each thread then
// quantises whole 32-output blocks of one row from 64 contiguous bytes and
// stores their 32 codes as two 16-byte writes.
template <class RowMap>
__device__ __forceinline__ void store_glu_q8(const Acc<L>& acc, uint8_t* lo, uint8_t* hi, uint8_t* hq,
                                             uint8_t* hqs, int f0, int F, float c, RowMap out_row) {
  static_assert(L::BM == 128 && L::BN / 2 == 256 && kStage >= 64 * 512, "tile of h in the ring");
  const int lane = threadIdx.x & 63, wn = wave_n<L>();
  const float inv_c = 1.0f / c;
#pragma unroll
  for (int j = 0; j < L::WN / 2; ++j) {
    const int fl = wn * glu_half_rows<L>() + j * 32 + (lane & 31);   // output within the tile
#pragma unroll
    for (int i = 0; i < L::WM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = acc_row<L>(i, r);
        if (out_row(tr) < 0) continue;   // padding rows: never read back
        bf16_t* row = (bf16_t*)((tr < 64 ? lo : hi) + (tr & 63) * 512);
        row[fl] = f32_to_bf16(situ_glu(acc.c[i][j][r], acc.c[i][j + L::WN / 2][r], c, inv_c));
      }
  }
  wg_barrier();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = (int)threadIdx.x + L::NT * u;   // 128 rows x 8 blocks = 2 per thread
    const int tr = q >> 3, b = q & 7;
    const int f = f0 + 32 * b;
    const int64_t orow = out_row(tr);
    if (orow < 0 || f >= F) continue;
    const uint4* src = (const uint4*)((tr < 64 ? lo : hi) + (tr & 63) * 512 + 64 * b);
    uint32_t w[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 x = src[v];
      w[4 * v] = x.x; w[4 * v + 1] = x.y; w[4 * v + 2] = x.z; w[4 * v + 3] = x.w;
    }
    float x[32];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
    const int X = ef == 0 ? -127 : max(-127, min(127, ef - 127 - 8));
    uint32_t code[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float y[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) y[t] = fminf(fmaxf(__builtin_ldexpf(x[4 * e + t] + 0.0f, -X), -448.0f), 448.0f);
      uint32_t p = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      code[e] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)p, true);
    }
    uint4* dst = (uint4*)(hq + orow * F + f);
    dst[0] = make_uint4(code[0], code[1], code[2], code[3]);
    dst[1] = make_uint4(code[4], code[5], code[6], code[7]);
    hqs[orow * (F / 32) + f / 32] = (uint8_t)(X + 127);
  }
}
}  // namespace mx8

// H[r] = act(zq[perm_src[r] / k] W_g[e]^T, ... W_v[e]^T) for the rows of expert e,
// zq in MXFP8 (codes Z, scales z_scale), W_g / W_v in MXFP4. With a.hq set the
// rows go out in MXFP8 (hq, hqs) instead of bf16 H.
template <int CP>
__global__ __launch_bounds__(512) void grouped_glu_mx8_kernel(GroupedGluArgs a) {
  using C = mx8::L;
  MOE_MX8_RING;
  const int ntn = (int)ceil_div(a.F, C::BN / 2);
  int64_t L;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, L)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<C::BM>(a.tile_info, ntn, a.rows_cap, L, e, nt, row_lo, row_hi);
  const int f0 = nt * (C::BN / 2);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  mx8::Src s;
  s.ra = make_rsrc(a.Z, (int64_t)a.T * a.ldz);
  s.rsa = make_rsrc(a.z_scale, (int64_t)a.T * (a.K / 32));
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = row_lo + 16 * w + 8 * q + (lane >> 3);
    uint32_t off = kOOB;
    if (row >= 0 && row < row_hi) {
      const int t = a.perm_src[row] / a.topk;
      if (a.perm_src[row] >= 0 && t < a.T) off = (uint32_t)((int64_t)t * a.ldz);
    }
    s.aoff[q] = off;
  }
  {
    const int row = row_lo + 16 * w + lane;
    uint32_t off = kOOB;
    if (lane < 16 && row >= 0 && row < row_hi) {
      const int t = a.perm_src[row] / a.topk;
      if (a.perm_src[row] >= 0 && t < a.T) off = (uint32_t)(t * (a.K / 32));
    }
    s.asoff = off;
  }
  mx8::b_src_glu(s, a.Wg, a.Wv, (int64_t)e * a.F, a.K, f0, a.F, a.w_tiled != 0);
  Acc<C> acc;
  acc_zero(acc);
  mx8::mainloop_rows<CP>(mx0, mx1, mx2, s, a.K, row_hi - row_lo, acc);
  const auto rowmap = [=](int tr) -> int64_t {
    const int r = row_lo + tr;
    return (r >= 0 && r < row_hi) ? (int64_t)r : -1;
  };
  if (a.hq != nullptr) mx8::store_glu_q8(acc, mx0, mx1, a.hq, a.hqs, f0, a.F, a.c, rowmap);
  else store_glu(acc, (bf16_t*)a.H, a.F, f0, a.F, a.c, rowmap);
}

// O[r] = hq[r] W_o[e]^T for the rows of expert e, hq in MXFP8 (codes H, scales
// h_scale), W_o in MXFP4.
template <int CP>
__global__ __launch_bounds__(512) void grouped_down_mx8_kernel(GroupedDownArgs a) {
  using C = mx8::L;
  MOE_MX8_RING;
  const int ntn = (int)ceil_div(a.N, C::BN);
  int64_t L;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, L)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<C::BM>(a.tile_info, ntn, a.rows_cap, L, e, nt, row_lo, row_hi);
  const int n0 = nt * C::BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lo = max(row_lo, 0), nrows = max(0, row_hi - lo);
  mx8::Src s;
  s.ra = make_rsrc((const uint8_t*)a.H + (int64_t)lo * a.ldh, (int64_t)nrows * a.ldh);
  s.rsa = make_rsrc(a.h_scale + (int64_t)lo * (a.K / 32), (int64_t)nrows * (a.K / 32));
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 16 * w + 8 * q + (lane >> 3);
    s.aoff[q] = r < nrows ? (uint32_t)((int64_t)r * a.ldh) : kOOB;
  }
  const int rs = 16 * w + lane;
  s.asoff = (lane < 16 && rs < nrows) ? (uint32_t)(rs * (a.K / 32)) : kOOB;
  mx8::b_src_plain(s, a.Wo, (int64_t)e * a.N, a.K, n0, a.N, a.w_tiled != 0);
  Acc<C> acc;
  acc_zero(acc);
  mx8::mainloop_rows<CP>(mx0, mx1, mx2, s, a.K, row_hi - row_lo, acc);
  store_tile(acc, (bf16_t*)a.O, a.N, row_lo, n0, row_hi, a.N);
}

// ---------------------------------------------------------------------------
// Grouped expert GEMMs with the weights in registers (bf16, fragment-tiled)
// ---------------------------------------------------------------------------
//
// The expert weights are re-laid once at load time (moe_bf16_tile) in the
// order the MFMA takes them: for each group of 32 weight rows and each k-step
// of 16, the 32 x 16 block as 64 lanes x 16 bytes, lane l holding row l % 32,
// k = 8 (l / 32) .. +7 (the B operand of v_mfma_f32_32x32x16_bf16); K padded to
// a multiple of 64 with zeros. One B fragment is then one fully used 1 KB load
// straight into registers: the weights never pass through LDS. Only the
// gathered z (or h) rows do, through a 4-stage ring of 64-k tiles (16 KB
// each), shared by the block's 4 waves.
//
// A block is 4 waves side by side in N, one per SIMD, each owning WM x WN
// fragments of 32 x 32 (Shape). Per 16-k step a wave reads its WM A fragments
// from LDS and takes its WN B fragments from registers for WM x WN MFMAs; the
// B fragments of k-step q + LEAD are loaded while k-step q computes, into a
// ring of LEAD + 1 register slots. Wide, the shape of every kernel here:
// 128 x 512 (4 x 4 fragments per wave, B 7 k-steps ahead). A 256 x 256 shape
// (8 x 2 fragments, B 15 k-steps ahead) ran the K3 prefill gate/up no faster
// (15.1 ms both) and the decode batch at 7.9 against 6.3 ms.
namespace bt {
constexpr int NW = 4, BK = 64, KS = BK / 16;
constexpr int NSA = 4;                     // A stages

template <int WM_, int WN_, int LEAD_, int CP_ = 0>
struct Shape {
  static constexpr int WM = WM_, WN = WN_, LEAD = LEAD_, SLOTS = LEAD_ + 1, CP = CP_;   // CP: weight loads
  static constexpr int BM = 32 * WM, BN = 32 * WN * NW;
  static constexpr int AR = BM / (NW * 8);          // A DMA per wave per stage (8 rows of 128 B)
  using L = Cfg<1, NW, WM, WN, BK, 2>;              // accumulator / epilogue layout
  static_assert(L::BM == BM && L::BN == BN && L::NT == 256 && L::AR == AR, "layout");
  static_assert((NSA * KS) % SLOTS == 0 && WN % 2 == 0, "slot ring; gate/up halves");
  // vector-memory ops issued after the DMA of the A stage that the end of
  // tile T (0 .. NSA-1 within a round) waits for: the later stages' DMAs and
  // the B loads of the tiles since. The first round issues fewer (its DMAs
  // all come before its B loads).
  static constexpr int vm_after_dma(int T, bool first) {
    return (NSA - 2) * AR + ((first && T + 1 < NSA - 1) ? T + 1 : NSA - 1) * KS * WN;
  }
};
using Wide = Shape<4, 4, 7>;
// 32 x 512 (one row fragment per wave) for the MXFP4 kernels at batches of few
// rows per expert
using Thin = Shape<1, 4, 7, kStream>;
constexpr int BM = Wide::BM, BN = Wide::BN, AR = Wide::AR;
using L = Wide::L;

template <int WN>
struct BSrc {
  rsrc_t r[2];                 // weight resources (gate, up for a GLU tile; one for plain)
  uint32_t off[WN];            // byte offset of fragment j's first k-step tile + 16 lane, or kOOB
};

// WN B fragments (one k-step) into slot registers: fragment j of k-step q is
// the 1 KB at off[j] + 1024 q (the second half of the fragments through r[1]).
template <int WN, int CP>
__device__ __forceinline__ void load_b(const BSrc<WN>& b, int q, bf16x8 (&dst)[WN]) {
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const uint32_t o = b.off[j];
    dst[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                            b.r[j >= WN / 2 ? 1 : 0], o + 1024u * (uint32_t)q, 0, CP));
  }
}

// A fragments of k-step ks of an A stage (BM x BK, the swizzled 128-byte rows
// of the DMA engine): NV fragments of 32 rows.
template <int NV, int WM>
__device__ __forceinline__ void read_a(const bf16_t* S, int ks, bf16x8 (&fa)[WM]) {
  if constexpr (NV > 0) {
    const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
    const bf16_t* Aw = S + lr * BK;
    const int slot = 8 * ((2 * ks + lh) ^ swz<L>(lr));
#pragma unroll
    for (int i = 0; i < NV; ++i) fa[i] = *(const bf16x8*)(Aw + i * 32 * BK + slot);
  }
}

template <int NV, class C>
__device__ __forceinline__ void mma_q(const bf16x8 (&fa)[C::WM], const bf16x8 (&fb)[C::WN], Acc<C>& acc) {
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j)
      acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc.c[i][j], 0, 0, 0);
}

template <class S>
__device__ __forceinline__ void dma_a(const Rows<S::AR>& ar, bf16_t* St, int kt, int K) {
  dma_rows<typename S::L, S::AR>(ar, St, kt * BK, K);
}

// B register slots: slot s holds the WN fragments of the k-steps q = s (mod SLOTS).
template <class S>
struct BRing {
  bf16x8 b[S::SLOTS][S::WN];
};

// One k-step Q (0 .. NSA KS - 1) of a round of NSA K-tiles (round base k-step
// q0): load B of k-step q0 + Q + LEAD, then (ks < KS-1) read the next A
// fragments of this tile or (ks == KS-1) wait for the next tile's stage,
// barrier, refill this stage with tile kt + NSA and read the next tile's first
// A fragments; then this k-step's MFMAs.
template <class S, int NV, int Q>
__device__ __forceinline__ void bt_kstep(bf16_t* const (&st)[NSA], const Rows<S::AR>& ar,
                                         const BSrc<S::WN>& bs, int q0, int K, BRing<S>& br,
                                         bf16x8 (&fa0)[S::WM], bf16x8 (&fa1)[S::WM],
                                         Acc<typename S::L>& acc) {
  constexpr int T = Q / KS, ks = Q % KS;
  constexpr int slot = Q % S::SLOTS, lslot = (Q + S::LEAD) % S::SLOTS;
  load_b<S::WN, S::CP>(bs, q0 + Q + S::LEAD, br.b[lslot]);
  if constexpr (ks + 1 < KS) {
    if constexpr (ks & 1) read_a<NV>(st[T], ks + 1, fa0);
    else read_a<NV>(st[T], ks + 1, fa1);
  } else {
    // the next tile's A stage must have landed (own DMA, then every wave's),
    // and every wave must be done reading this stage before it is refilled;
    // the B loads issued since that DMA stay in flight.
    if (q0 == 0) __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0_vm(S::vm_after_dma(T, true)));
    else __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0_vm(S::vm_after_dma(T, false)));
    wg_barrier();
    dma_a<S>(ar, st[T], (q0 / KS) + T + NSA, K);
    static_assert(KS % 2 == 0, "k-step 0 of a tile reads into fa0");
    read_a<NV>(st[(T + 1) % NSA], 0, fa0);
  }
  if constexpr (ks & 1) mma_q<NV, typename S::L>(fa1, br.b[slot], acc);
  else mma_q<NV, typename S::L>(fa0, br.b[slot], acc);
  // one wave per SIMD: the next k-step's A reads and the loads go between the
  // MFMAs, so that their latency overlaps matrix work. Per A fragment i:
  // MFMA, read, MFMA, one load (the B loads before the tile's barrier, the
  // refill DMA of the A stage after it), the other MFMAs.
  if constexpr (NV > 0) {
    constexpr int V = ks + 1 < KS ? S::WN : S::AR;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < V) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if constexpr (S::WN > 2) __builtin_amdgcn_sched_group_barrier(0x008, S::WN - 2, 0);
    }
  }
}

template <class S, int NV, int Q>
__device__ __forceinline__ void bt_round(bf16_t* const (&st)[NSA], const Rows<S::AR>& ar,
                                         const BSrc<S::WN>& bs, int q0, int K, BRing<S>& br,
                                         bf16x8 (&fa0)[S::WM], bf16x8 (&fa1)[S::WM],
                                         Acc<typename S::L>& acc) {
  if constexpr (Q < NSA * KS) {
    bt_kstep<S, NV, Q>(st, ar, bs, q0, K, br, fa0, fa1, acc);
    bt_round<S, NV, Q + 1>(st, ar, bs, q0, K, br, fa0, fa1, acc);
  }
}

template <class S, int NV>
__device__ __forceinline__ void bt_mainloop(bf16_t* const (&st)[NSA], const Rows<S::AR>& ar,
                                            const BSrc<S::WN>& bs, int K, Acc<typename S::L>& acc) {
  const int nq = (int)ceil_div(K, BK) * KS;       // k-steps, whole K-tiles
  BRing<S> br;
  // B of k-steps 0 .. LEAD-1, then A of tiles 0 .. NSA-1
#pragma unroll
  for (int q = 0; q < S::LEAD; ++q) load_b<S::WN, S::CP>(bs, q, br.b[q]);
#pragma unroll
  for (int t = 0; t < NSA; ++t) dma_a<S>(ar, st[t], t, K);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(S::AR * (NSA - 1)));
  wg_barrier();
  bf16x8 fa0[S::WM], fa1[S::WM];
  read_a<NV>(st[0], 0, fa0);
  // whole rounds of NSA K-tiles (tiles past K are zeros on both operands)
  for (int q0 = 0; q0 < nq; q0 += NSA * KS) bt_round<S, NV, 0>(st, ar, bs, q0, K, br, fa0, fa1, acc);
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();
}

// bt_mainloop with NV = the number of this block's 32-row fragments that hold
// valid rows (one instantiation per count).
template <class S, int NV = S::WM>
__device__ __forceinline__ void bt_mainloop_rows(bf16_t* const (&st)[NSA], const Rows<S::AR>& ar,
                                                 const BSrc<S::WN>& bs, int K, int valid_rows,
                                                 Acc<typename S::L>& acc) {
  if constexpr (NV == 0) {
    bt_mainloop<S, 0>(st, ar, bs, K, acc);
  } else {
    const int nv = __builtin_amdgcn_readfirstlane(max(0, min(S::WM, (valid_rows + 31) / 32)));
    if (nv >= NV) bt_mainloop<S, NV>(st, ar, bs, K, acc);
    else bt_mainloop_rows<S, NV - 1>(st, ar, bs, K, valid_rows, acc);
  }
}

// Byte offset, in the tiled layout of a weight with K padded to Kp (a
// multiple of 64), of this lane's 16 bytes of k-step 0 of the 32-row group
// holding row r (r % 32 == 0).
__device__ __forceinline__ uint32_t tiled_off(int r, int Kp) {
  return (uint32_t)(r / 32) * (uint32_t)(Kp / 16) * 1024u + 16u * (uint32_t)(threadIdx.x & 63);
}

// MXFP4 weights in the fragment order (moe_mxfp4_frag_tile), decoded in
// registers. Packed codes: per group g of 32 rows and 64-k tile t, 1 KB of 64
// lanes x 16 bytes; lane l (row 32 g + l % 32) holds in dword s the 8 codes of
// k-step s (k = 64 t + 16 s + 8 (l / 32) .. +7, low nibble first). Scales: per
// group g and 128-k pair p, 32 rows x 4 bytes (the e8m0 scales of the 32-element
// k-blocks 4 p .. 4 p + 3). K is padded to a multiple of 128 with code 0 and
// scale byte 0 (zeros). A k-step's 8 codes decode to the bf16 B fragment with
// four v_cvt_scalef32_pk_bf16_fp4 (exact: a power-of-two scaling of a 2-bit
// significand), the same values the row-major MXFP4 path stages in LDS.
struct MxSrc {
  rsrc_t rp[2], rs[2];           // packed codes, scales (gate, up; or one weight twice)
  uint32_t poff[4], soff[4];     // fragment j: byte offset of tile / pair 0 for this lane, or kOOB
};
constexpr int TSLOTS = 4, LEADT = 3;   // packed tiles in registers; tiles loaded ahead

struct MxRing {
  uint4 p[TSLOTS][4];            // packed codes of a tile, per fragment
  uint32_t sc[2][4];             // scale dwords of a tile pair, per fragment
};

template <int CP>
__device__ __forceinline__ void load_mx_tile(const MxSrc& m, int t, uint4 (&dst)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    dst[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           m.rp[j >= 2 ? 1 : 0], m.poff[j] + 1024u * (uint32_t)t, 0, CP));
}
template <int CP>
__device__ __forceinline__ void load_mx_scales(const MxSrc& m, int pr, uint32_t (&dst)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    dst[j] = __builtin_amdgcn_raw_buffer_load_b32(m.rs[j >= 2 ? 1 : 0], m.soff[j] + 128u * (uint32_t)pr, 0, CP);
}

// bf16 B fragments of one k-step from 8 e2m1 codes (a dword) and their e8m0 scale byte.
__device__ __forceinline__ bf16x8 decode_frag(uint32_t codes, uint32_t sbyte) {
  const float scale = sbyte == 0u ? 0x1p-127f : __uint_as_float(sbyte << 23);
  const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  const uint32_t w2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  const uint32_t w3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  return __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
}

// Decoded fragments of k-step ks of the tile in packed slot PS (scale slot SS,
// tile parity TP).
template <int PS, int SS, int TP, int KSI>
__device__ __forceinline__ void decode_kstep(const MxRing& r, bf16x8 (&fb)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 q = r.p[PS][j];
    const uint32_t codes = KSI == 0 ? q.x : KSI == 1 ? q.y : KSI == 2 ? q.z : q.w;
    const uint32_t sbyte = (r.sc[SS][j] >> (8 * (2 * TP + KSI / 2))) & 0xFFu;
    fb[j] = decode_frag(codes, sbyte);
  }
}

// One k-step Q (0 .. 15) of a round of NSA K-tiles on MXFP4 B: as bt_kstep, with
// the packed codes of tile kt + LEADT (and, at even tiles, the scales of the
// pair after the current one) loaded at each tile's first k-step, and the
// next k-step's B fragments decoded while this one's MFMAs run.
template <class S, int NV, int Q>
__device__ __forceinline__ void btmx_kstep(bf16_t* const (&st)[NSA], const Rows<S::AR>& ar, const MxSrc& ms,
                                           int q0, int K, MxRing& mr, bf16x8 (&fa0)[S::WM],
                                           bf16x8 (&fa1)[S::WM], bf16x8 (&fb0)[4], bf16x8 (&fb1)[4],
                                           Acc<typename S::L>& acc) {
  static_assert(S::WN == 4, "four B fragments per wave");
  constexpr int T = Q / KS, ks = Q % KS;
  const int t0 = q0 / KS;                              // first tile of the round (a multiple of 4)
  constexpr int QN = Q + 1, TN = (QN / KS) % NSA, KN = QN % KS;   // the next k-step
  if constexpr (ks == 0) {
    load_mx_tile<S::CP>(ms, t0 + T + LEADT, mr.p[(T + LEADT) % TSLOTS]);
    if constexpr (T % 2 == 0) load_mx_scales<S::CP>(ms, (t0 + T) / 2 + 1, mr.sc[(T / 2 + 1) % 2]);
  }
  // next k-step's B fragments (the next tile's first when ks == 3)
  if constexpr (ks & 1) decode_kstep<TN % TSLOTS, (TN / 2) % 2, TN % 2, KN>(mr, fb0);
  else decode_kstep<TN % TSLOTS, (TN / 2) % 2, TN % 2, KN>(mr, fb1);
  if constexpr (ks + 1 < KS) {
    if constexpr (ks & 1) read_a<NV>(st[T], ks + 1, fa0);
    else read_a<NV>(st[T], ks + 1, fa1);
  } else {
    // as in bt_kstep; the count is that of the first tile of the first round
    // (the A DMAs of tiles 2 and 3, then tile 0's codes and the second pair's
    // scales), which later tiles exceed, so they wait a little longer than
    // needed
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0_vm((NSA - 2) * S::AR + 8));
    wg_barrier();
    dma_a<S>(ar, st[T], t0 + T + NSA, K);
    read_a<NV>(st[(T + 1) % NSA], 0, fa0);
  }
  if constexpr (ks & 1) mma_q<NV>(fa1, fb1, acc);
  else mma_q<NV>(fa0, fb0, acc);
  if constexpr (NV > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NV, 0);
      if (i < NV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
    }
  }
}

template <class S, int NV, int Q>
__device__ __forceinline__ void btmx_round(bf16_t* const (&st)[NSA], const Rows<S::AR>& ar, const MxSrc& ms,
                                           int q0, int K, MxRing& mr, bf16x8 (&fa0)[S::WM],
                                           bf16x8 (&fa1)[S::WM], bf16x8 (&fb0)[4], bf16x8 (&fb1)[4],
                                           Acc<typename S::L>& acc) {
  if constexpr (Q < NSA * KS) {
    btmx_kstep<S, NV, Q>(st, ar, ms, q0, K, mr, fa0, fa1, fb0, fb1, acc);
    btmx_round<S, NV, Q + 1>(st, ar, ms, q0, K, mr, fa0, fa1, fb0, fb1, acc);
  }
}

template <class S, int NV>
__device__ __forceinline__ void btmx_mainloop(bf16_t* const (&st)[NSA], const Rows<S::AR>& ar, const MxSrc& ms,
                                              int K, Acc<typename S::L>& acc) {
  static_assert(NSA % TSLOTS == 0 && LEADT < TSLOTS && NSA % 2 == 0, "slot rings");
  const int nq = (int)ceil_div(K, BK) * KS;
  MxRing mr;
  load_mx_tile<S::CP>(ms, 0, mr.p[0]);
  load_mx_tile<S::CP>(ms, 1, mr.p[1]);
  load_mx_tile<S::CP>(ms, 2, mr.p[2]);
  static_assert(LEADT == 3, "prologue");
  load_mx_scales<S::CP>(ms, 0, mr.sc[0]);
#pragma unroll
  for (int t = 0; t < NSA; ++t) dma_a<S>(ar, st[t], t, K);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(S::AR * (NSA - 1)));
  wg_barrier();
  bf16x8 fa0[S::WM], fa1[S::WM], fb0[4], fb1[4];
  read_a<NV>(st[0], 0, fa0);
  decode_kstep<0, 0, 0, 0>(mr, fb0);
  for (int q0 = 0; q0 < nq; q0 += NSA * KS)
    btmx_round<S, NV, 0>(st, ar, ms, q0, K, mr, fa0, fa1, fb0, fb1, acc);
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();
}

// btmx_mainloop with NV = the number of this block's 32-row fragments that
// hold valid rows (one instantiation per count).
template <class S, int NV = S::WM>
__device__ __forceinline__ void btmx_mainloop_rows(bf16_t* const (&st)[NSA], const Rows<S::AR>& ar,
                                                   const MxSrc& ms, int K, int valid_rows,
                                                   Acc<typename S::L>& acc) {
  if constexpr (NV == 0) {
    btmx_mainloop<S, 0>(st, ar, ms, K, acc);
  } else {
    const int nv = __builtin_amdgcn_readfirstlane(max(0, min(S::WM, (valid_rows + 31) / 32)));
    if (nv >= NV) btmx_mainloop<S, NV>(st, ar, ms, K, acc);
    else btmx_mainloop_rows<S, NV - 1>(st, ar, ms, K, valid_rows, acc);
  }
}

// Byte offsets, in the fragment-tiled MXFP4 layout of a weight with K padded
// to Kp (a multiple of 128), of this lane's packed 16 bytes of tile 0 and its
// scale dword of pair 0, for the 32-row group holding row r (r % 32 == 0).
__device__ __forceinline__ uint32_t mx_tiled_poff(int r, int Kp) {
  return (uint32_t)(r / 32) * (uint32_t)(Kp / 64) * 1024u + 16u * (uint32_t)(threadIdx.x & 63);
}
__device__ __forceinline__ uint32_t mx_tiled_soff(int r, int Kp) {
  return (uint32_t)(r / 32) * (uint32_t)(Kp / 128) * 128u + 4u * (uint32_t)(threadIdx.x & 31);
}

// the A ring of a register-B block of ROWS rows: NSA stages of ROWS x BK bf16
#define MOE_BT_RING(ROWS)                                       \
  __shared__ __align__(16) bf16_t la0[(ROWS) * bt::BK];          \
  __shared__ __align__(16) bf16_t la1[(ROWS) * bt::BK];          \
  __shared__ __align__(16) bf16_t la2[(ROWS) * bt::BK];          \
  __shared__ __align__(16) bf16_t la3[(ROWS) * bt::BK];          \
  bf16_t* const st[bt::NSA] = {la0, la1, la2, la3}
static_assert(NSA == 4, "ring arrays");
}  // namespace bt

// grouped_glu on tiled bf16 weights: H[r] = act(z W_g[e]^T, z W_v[e]^T) for the
// rows of expert e, BN/2 outputs per block (wave w: outputs f0 + w BN/8 + 0 ..
// BN/8 - 1; its first WN/2 fragments gate, the others up).
__global__ __launch_bounds__(bt::NW * 64) void grouped_glu_bt_kernel(GroupedGluArgs a) {
  using namespace bt;
  using S = Wide;
  using C = S::L;
  MOE_BT_RING(S::BM);
  const int ntn = (int)ceil_div(a.F, S::BN / 2);
  int64_t Li;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, Li)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<S::BM>(a.tile_info, ntn, a.rows_cap, Li, e, nt, row_lo, row_hi);
  const int f0 = nt * (S::BN / 2);
  Rows<S::AR> ar;
  ar.r[0] = ar.r[1] = make_rsrc(a.Z, (int64_t)a.T * a.ldz * 2);
#pragma unroll
  for (int q = 0; q < S::AR; ++q) {
    ar.sel[q] = 0;
    const int row = row_lo + dma_row<C, S::AR>(q);
    uint32_t off = kOOB;
    if (row >= 0 && row < row_hi) {
      const int src = a.perm_src[row];
      const int t = src / a.topk;
      if (src >= 0 && t < a.T) off = (uint32_t)((int64_t)t * a.ldz * 2);
    }
    ar.off[q] = off;
  }
  const int Kp = (int)ceil_div(a.K, BK) * BK;
  const int64_t ebytes = (int64_t)a.F * Kp * 2;                 // one expert's tiled weight
  BSrc<S::WN> bs;
  bs.r[0] = make_rsrc((const uint8_t*)a.Wg.data + e * ebytes, ebytes);
  bs.r[1] = make_rsrc((const uint8_t*)a.Wv.data + e * ebytes, ebytes);
  const int w = threadIdx.x >> 6;
  constexpr int H = S::WN / 2;                                   // gate (= up) fragments per wave
#pragma unroll
  for (int j = 0; j < S::WN; ++j) {
    const int f = f0 + 32 * H * w + 32 * (j % H);
    bs.off[j] = f < a.F ? tiled_off(f, Kp) : kOOB;
  }
  Acc<C> acc;
  acc_zero(acc);
  bt_mainloop_rows<S>(st, ar, bs, a.K, row_hi - row_lo, acc);
  store_glu(acc, (bf16_t*)a.H, a.F, f0, a.F, a.c, [=](int tr) -> int64_t {
    const int r = row_lo + tr;
    return (r >= 0 && r < row_hi) ? (int64_t)r : -1;
  });
}

// grouped_down on tiled bf16 weights: O[r] = H[r] W_o[e]^T, BN outputs per block.
__global__ __launch_bounds__(bt::NW * 64) void grouped_down_bt_kernel(GroupedDownArgs a) {
  using namespace bt;
  using S = Wide;
  using C = S::L;
  MOE_BT_RING(S::BM);
  const int ntn = (int)ceil_div(a.N, S::BN);
  int64_t Li;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, Li)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<S::BM>(a.tile_info, ntn, a.rows_cap, Li, e, nt, row_lo, row_hi);
  const int n0 = nt * S::BN;
  const Rows<S::AR> ar = a_rows_dense<C, S::AR>(a.H, a.ldh, max(row_lo, 0), max(row_hi, 0));
  const int Kp = (int)ceil_div(a.K, BK) * BK;
  const int64_t ebytes = (int64_t)a.N * Kp * 2;
  BSrc<S::WN> bs;
  bs.r[0] = bs.r[1] = make_rsrc((const uint8_t*)a.Wo.data + e * ebytes, ebytes);
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < S::WN; ++j) {
    const int n = n0 + (S::BN / NW) * w + 32 * j;
    bs.off[j] = n < a.N ? tiled_off(n, Kp) : kOOB;
  }
  Acc<C> acc;
  acc_zero(acc);
  bt_mainloop_rows<S>(st, ar, bs, a.K, row_hi - row_lo, acc);
  store_tile(acc, (bf16_t*)a.O, a.N, row_lo, n0, row_hi, a.N);
}

// grouped_glu_bt on fragment-tiled MXFP4 weights (decoded in registers), on
// block shape S (Wide: 128 rows; Thin: 32 rows, for few rows per expert).
template <class S>
__global__ __launch_bounds__(bt::NW * 64) void grouped_glu_btmx_kernel(GroupedGluArgs a) {
  using namespace bt;
  using C = typename S::L;
  MOE_BT_RING(S::BM);
  const int ntn = (int)ceil_div(a.F, S::BN / 2);
  int64_t Li;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, Li)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<S::BM>(a.tile_info, ntn, a.rows_cap, Li, e, nt, row_lo, row_hi);
  const int f0 = nt * (S::BN / 2);
  Rows<S::AR> ar;
  ar.r[0] = ar.r[1] = make_rsrc(a.Z, (int64_t)a.T * a.ldz * 2);
#pragma unroll
  for (int q = 0; q < S::AR; ++q) {
    ar.sel[q] = 0;
    const int row = row_lo + dma_row<C, S::AR>(q);
    uint32_t off = kOOB;
    if (row >= 0 && row < row_hi) {
      const int src = a.perm_src[row];
      const int t = src / a.topk;
      if (src >= 0 && t < a.T) off = (uint32_t)((int64_t)t * a.ldz * 2);
    }
    ar.off[q] = off;
  }
  const int Kp = (int)ceil_div(a.K, 128) * 128;
  const int64_t pbytes = (int64_t)a.F * Kp / 2, sbytes = (int64_t)a.F * Kp / 32;   // one expert
  MxSrc ms;
  ms.rp[0] = make_rsrc((const uint8_t*)a.Wg.data + e * pbytes, pbytes);
  ms.rp[1] = make_rsrc((const uint8_t*)a.Wv.data + e * pbytes, pbytes);
  ms.rs[0] = make_rsrc(a.Wg.scale + e * sbytes, sbytes);
  ms.rs[1] = make_rsrc(a.Wv.scale + e * sbytes, sbytes);
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int f = f0 + 64 * w + 32 * (j & 1);
    ms.poff[j] = f < a.F ? mx_tiled_poff(f, Kp) : kOOB;
    ms.soff[j] = f < a.F ? mx_tiled_soff(f, Kp) : kOOB;
  }
  Acc<C> acc;
  acc_zero(acc);
  btmx_mainloop_rows<S>(st, ar, ms, a.K, row_hi - row_lo, acc);
  store_glu(acc, (bf16_t*)a.H, a.F, f0, a.F, a.c, [=](int tr) -> int64_t {
    const int r = row_lo + tr;
    return (r >= 0 && r < row_hi) ? (int64_t)r : -1;
  });
}

template <class S>
__global__ __launch_bounds__(bt::NW * 64) void grouped_down_btmx_kernel(GroupedDownArgs a) {
  using namespace bt;
  using C = typename S::L;
  MOE_BT_RING(S::BM);
  const int ntn = (int)ceil_div(a.N, S::BN);
  int64_t Li;
  if (!xcd_item((int64_t)__builtin_amdgcn_readfirstlane(a.tile_off[a.E]) * ntn, Li)) return;
  int e, nt, row_lo, row_hi;
  grouped_item<S::BM>(a.tile_info, ntn, a.rows_cap, Li, e, nt, row_lo, row_hi);
  const int n0 = nt * S::BN;
  const Rows<S::AR> ar = a_rows_dense<C, S::AR>(a.H, a.ldh, max(row_lo, 0), max(row_hi, 0));
  const int Kp = (int)ceil_div(a.K, 128) * 128;
  const int64_t pbytes = (int64_t)a.N * Kp / 2, sbytes = (int64_t)a.N * Kp / 32;
  MxSrc ms;
  ms.rp[0] = ms.rp[1] = make_rsrc((const uint8_t*)a.Wo.data + e * pbytes, pbytes);
  ms.rs[0] = ms.rs[1] = make_rsrc(a.Wo.scale + e * sbytes, sbytes);
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 128 * w + 32 * j;
    ms.poff[j] = n < a.N ? mx_tiled_poff(n, Kp) : kOOB;
    ms.soff[j] = n < a.N ? mx_tiled_soff(n, Kp) : kOOB;
  }
  Acc<C> acc;
  acc_zero(acc);
  btmx_mainloop_rows<S>(st, ar, ms, a.K, row_hi - row_lo, acc);
  store_tile(acc, (bf16_t*)a.O, a.N, row_lo, n0, row_hi, a.N);
}

// Fragment-tiled copy of a row-major MXFP4 weight (packed [rows, K/2], scales
// [rows, K/32]; rows % 32 == 0, K % 32 == 0), K padded to Kp = ceil(K / 128)
// 128: one thread per output dword of the packed codes (lane l's dword s of
// tile t of group g: the 4 bytes of row 32 g + l % 32 holding k = 64 t + 16 s +
// 8 (l / 32) .. +7), and one per output scale dword (4 scales of a row).
__global__ __launch_bounds__(256) void tile_mxfp4_frag_kernel(const uint8_t* __restrict__ packed,
                                                              const uint8_t* __restrict__ scale,
                                                              uint32_t* __restrict__ pout,
                                                              uint32_t* __restrict__ sout, int64_t rows,
                                                              int K, int Kp) {
  const int64_t np = rows / 32 * (Kp / 64) * 256;       // dwords of packed codes
  const int64_t ns = rows * (Kp / 128);                 // scale dwords
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < np + ns;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (i < np) {
      const int sdw = (int)(i & 3), lane = (int)((i >> 2) & 63);
      const int64_t tile = i >> 8;
      const int t = (int)(tile % (Kp / 64));
      const int64_t g = tile / (Kp / 64);
      const int64_t r = g * 32 + (lane & 31);
      const int k = 64 * t + 16 * sdw + 8 * (lane >> 5);     // 8 codes = 4 bytes from k / 2
      uint32_t v = 0;
      if (k < K) v = *(const uint32_t*)(packed + r * (K / 2) + k / 2);   // K % 32: all 8 in or out
      pout[i] = v;
    } else {
      const int64_t j = i - np;                          // (g, pair, row-in-group) order
      const int rl = (int)(j & 31);
      const int64_t gp = j >> 5;
      const int pr = (int)(gp % (Kp / 128));
      const int64_t g = gp / (Kp / 128);
      const int64_t r = g * 32 + rl;
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int kb = 4 * pr + b;                       // 32-element block
        if (kb < K / 32) v |= (uint32_t)scale[r * (K / 32) + kb] << (8 * b);
      }
      sout[j] = v;
    }
  }
}

// Fragment-tiled copy of a bf16 weight [rows, K] (rows % 32 == 0): one thread
// per 16-byte piece of the output; K padded to Kp = ceil(K / 64) 64 with zeros.
__global__ __launch_bounds__(256) void tile_bf16_kernel(const bf16_t* __restrict__ in, uint4* __restrict__ out,
                                                        int64_t rows, int K, int Kp) {
  const int64_t n = rows / 32 * (Kp / 16) * 64;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    const int64_t tile = i >> 6;
    const int s = (int)(tile % (Kp / 16));
    const int64_t g = tile / (Kp / 16);
    const int64_t r = g * 32 + (lane & 31);
    const int k = 16 * s + 8 * (lane >> 5);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k < K) v = *(const uint4*)(in + r * K + k);      // K % 8 == 0: a piece is all in or all out
    out[i] = v;
  }
}

}  // namespace

int launch_tile_bf16(const void* in, void* out, int64_t rows, int K, hipStream_t stream) {
  if (rows % 32 || K % 8 || ((uintptr_t)in | (uintptr_t)out) % 16) return -1;
  if (rows == 0) return 0;
  const int Kp = (int)ceil_div(K, bt::BK) * bt::BK;
  const int64_t n = rows / 32 * (Kp / 16) * 64;
  hipLaunchKernelGGL(tile_bf16_kernel, dim3((unsigned)(ceil_div(n, 256) < 16384 ? ceil_div(n, 256) : 16384)),
                     dim3(256), 0, stream, (const bf16_t*)in, (uint4*)out, rows, K, Kp);
  return (int)hipGetLastError();
}

int64_t tiled_bf16_bytes(int64_t rows, int K) { return rows * (ceil_div(K, bt::BK) * bt::BK) * 2; }

int launch_tile_mxfp4_frag(const uint8_t* data, const uint8_t* scale, uint8_t* data_out, uint8_t* scale_out,
                           int64_t rows, int K, hipStream_t stream) {
  if (rows % 32 || K % 32 || ((uintptr_t)data_out | (uintptr_t)scale_out) % 4 || (uintptr_t)data % 4)
    return -1;
  if (rows == 0) return 0;
  const int Kp = (int)ceil_div(K, 128) * 128;
  const int64_t n = rows / 32 * (Kp / 64) * 256 + rows * (Kp / 128);
  hipLaunchKernelGGL(tile_mxfp4_frag_kernel, dim3((unsigned)(ceil_div(n, 256) < 16384 ? ceil_div(n, 256) : 16384)),
                     dim3(256), 0, stream, data, scale, (uint32_t*)data_out, (uint32_t*)scale_out, rows, K, Kp);
  return (int)hipGetLastError();
}

void tiled_mxfp4_frag_bytes(int64_t rows, int K, int64_t* data_bytes, int64_t* scale_bytes) {
  const int64_t Kp = ceil_div(K, 128) * 128;
  *data_bytes = rows * Kp / 2;
  *scale_bytes = rows * Kp / 32;
}

// Below 256 single-pass tiles the chip is not full: take 128 x 128 tiles and
// split K until about 256 blocks run, each over at least 6 K-tiles.
SplitK plan_split(int act_dtype, int M, int ncols, int K) {
  SplitK p;
  if (act_dtype != DT_BF16 || M == 0) return p;
  if (ceil_div(M, DenseCfg::BM) * ceil_div(ncols, DenseCfg::BN) >= 256) return p;
  const int64_t tiles = ceil_div(M, SplitCfg::BM) * ceil_div(ncols, SplitCfg::BN);
  int s = 1;
  while (s < 16 && tiles * s < 256 && K / (2 * s) >= 6 * SplitCfg::BK) s *= 2;
  const int unit = SplitCfg::NS * SplitCfg::BK;  // the ring walks K-tiles NS at a time
  p.kchunk = (int)(ceil_div(ceil_div(K, s), unit) * unit);
  p.splits = (int)ceil_div(K, p.kchunk);
  return p;
}

int multiseg_slices(int act_dtype, int M, int N, int nseg) {
  if (act_dtype != DT_BF16 || M == 0 || nseg < 2) return 0;
  if (ceil_div(M, DenseCfg::BM) * ceil_div(N, DenseCfg::BN) >= 256) return 0;
  return nseg;
}

// Row tiles of the grouped expert GEMMs: 1 on the fp32 path; 128 on the
// scaled-MFMA path and with MXFP4 weights; with bf16 weights, 320 (the
// pipelined big tiles) once the experts average at least kBigRows rows, else
// 128 (at decode sizes the weight stream sets the pace and the smaller tiles
// waste no DMA on padding rows). Fragment-tiled MXFP4 weights: 32-row tiles
// while the experts average fewer than kThinRows rows, else 128.
#ifndef MOE_BIG_ROWS
#define MOE_BIG_ROWS 64
#endif
#ifndef MOE_THIN_ROWS
#define MOE_THIN_ROWS 16
#endif
constexpr int kBigRows = MOE_BIG_ROWS, kThinRows = MOE_THIN_ROWS;
int grouped_bm(int act_dtype, int expert_w_dtype, int act_mx8, int w_tiled, int64_t rows, int E) {
  if (act_dtype == DT_F32) return 1;
  if (act_mx8) return mx8::L::BM;
  if (w_tiled && expert_w_dtype == DT_MXFP4)
    return rows < (int64_t)kThinRows * E ? bt::Thin::BM : bt::Wide::BM;
  if (w_tiled) return bt::BM;         // fragment-tiled bf16 weights
  if (expert_w_dtype == DT_BF16 && rows >= (int64_t)kBigRows * E) return GroupBigCfg::BM;
  return GroupCfg::BM;
}

int launch_dense(const DenseArgs& a, hipStream_t stream) {
  if (a.act_dtype == DT_F32) return launch_dense_f32(a, stream);
  if (a.M == 0) return 0;
  if (a.split.splits > 0) {
    using C = SplitCfg;
    dim3 grid((unsigned)xcd_grid(ceil_div(a.N, C::BN) * ceil_div(a.M, C::BM) * a.split.splits));
    if (a.W.dtype == DT_MXFP4) hipLaunchKernelGGL(dense_split_kernel<true>, grid, dim3(SplitCfg::NT), 0, stream, a);
    else hipLaunchKernelGGL(dense_split_kernel<false>, grid, dim3(SplitCfg::NT), 0, stream, a);
    const int64_t n4 = (int64_t)a.M * a.N / 4;
    hipLaunchKernelGGL(reduce_store_kernel, dim3(reduce_blocks(n4)), dim3(256), 0, stream, a.P,
                       a.split.splits, a.M, a.N, (bf16_t*)a.C, a.ldc);
    return (int)hipGetLastError();
  }
  if (a.W.dtype != DT_BF16) return -1;   // MXFP4: decode to bf16 first (launch_decode_mxfp4)
  using C = DenseCfg;
  dim3 grid((unsigned)xcd_grid(ceil_div(a.N, C::BN) * ceil_div(a.M, C::BM)));
  hipLaunchKernelGGL(dense_kernel, grid, dim3(DenseCfg::NT), 0, stream, a);
  return (int)hipGetLastError();
}

int launch_glu(const GluArgs& a, hipStream_t stream) {
  if (a.act_dtype == DT_F32) return launch_glu_f32(a, stream);
  if (a.M == 0) return 0;
  if (a.Wg.dtype != DT_BF16 || a.Wv.dtype != DT_BF16) return -1;   // the shared experts are bf16
  if (a.split.splits > 0) {
    using C = SplitCfg;
    dim3 grid((unsigned)xcd_grid(ceil_div(a.F, C::BN / 2) * ceil_div(a.M, C::BM) * a.split.splits));
    hipLaunchKernelGGL(glu_split_kernel, grid, dim3(SplitCfg::NT), 0, stream, a);
    const int64_t n4 = (int64_t)a.M * a.F / 4;
    hipLaunchKernelGGL(reduce_glu_kernel, dim3(reduce_blocks(n4)), dim3(256), 0, stream, a.P,
                       a.split.splits, a.M, a.F, a.c, (bf16_t*)a.H, a.ldh);
    return (int)hipGetLastError();
  }
  using C = DenseCfg;
  dim3 grid((unsigned)xcd_grid(ceil_div(a.F, C::BN / 2) * ceil_div(a.M, C::BM)));
  hipLaunchKernelGGL(glu_kernel, grid, dim3(DenseCfg::NT), 0, stream, a);
  return (int)hipGetLastError();
}

int launch_grouped_glu(const GroupedGluArgs& a, hipStream_t stream) {
  if (a.act_dtype == DT_F32) return launch_grouped_glu_f32(a, stream);
  if (a.max_tiles == 0) return 0;
  if (a.act_mx8) {
    if (a.bm != mx8::L::BM || a.Wg.dtype != DT_MXFP4 || a.K % mx8::kBK) return -1;
    if (a.w_tiled && (a.F % 64 || mx8::kBRW != 64)) return -1;
    // h goes either to bf16 H or, as MXFP8, to hq and hqs: never to neither
    if (a.hq != nullptr ? a.hqs == nullptr : a.H == nullptr) return -1;
    dim3 grid((unsigned)xcd_grid(ceil_div(a.F, mx8::L::BN / 2) * a.max_tiles));
    if (a.rows_cap < (int64_t)kThinRows * a.E)   // weight slices read once: stream them
      hipLaunchKernelGGL(grouped_glu_mx8_kernel<kStream>, grid, dim3(mx8::L::NT), 0, stream, a);
    else
      hipLaunchKernelGGL(grouped_glu_mx8_kernel<0>, grid, dim3(mx8::L::NT), 0, stream, a);
    return (int)hipGetLastError();
  }
  if (a.H == nullptr) return -1;
  if (a.w_tiled) {
    dim3 grid((unsigned)xcd_grid(ceil_div(a.F, bt::BN / 2) * a.max_tiles));   // BN: every shape's
    static_assert(bt::Thin::BN == bt::BN && bt::Wide::BN == bt::BN, "one n-tile width");
    if (a.Wg.dtype == DT_MXFP4 && a.bm == bt::Thin::BM)
      hipLaunchKernelGGL(grouped_glu_btmx_kernel<bt::Thin>, grid, dim3(bt::NW * 64), 0, stream, a);
    else if (a.Wg.dtype == DT_MXFP4 && a.bm == bt::Wide::BM)
      hipLaunchKernelGGL(grouped_glu_btmx_kernel<bt::Wide>, grid, dim3(bt::NW * 64), 0, stream, a);
    else if (a.Wg.dtype == DT_BF16 && a.bm == bt::BM)
      hipLaunchKernelGGL(grouped_glu_bt_kernel, grid, dim3(bt::NW * 64), 0, stream, a);
    else
      return -1;
    return (int)hipGetLastError();
  }
  if (a.bm == GroupBigCfg::BM && a.bm != GroupCfg::BM) {
    if (a.Wg.dtype != DT_BF16) return -1;
    dim3 grid((unsigned)xcd_grid(ceil_div(a.F, GroupBigCfg::BN / 2) * a.max_tiles));
    hipLaunchKernelGGL(grouped_glu_big_kernel, grid, dim3(GroupBigCfg::NT), 0, stream, a);
    return (int)hipGetLastError();
  }
  if (a.bm != GroupCfg::BM) return -1;
  using C = GroupCfg;
  dim3 grid((unsigned)xcd_grid(ceil_div(a.F, C::BN / 2) * a.max_tiles));
  if (a.Wg.dtype == DT_MXFP4) hipLaunchKernelGGL(grouped_glu_kernel<true>, grid, dim3(C::NT), 0, stream, a);
  else hipLaunchKernelGGL(grouped_glu_kernel<false>, grid, dim3(C::NT), 0, stream, a);
  return (int)hipGetLastError();
}

int launch_grouped_down(const GroupedDownArgs& a, hipStream_t stream) {
  if (a.act_dtype == DT_F32) return launch_grouped_down_f32(a, stream);
  if (a.max_tiles == 0) return 0;
  if (a.act_mx8) {
    if (a.bm != mx8::L::BM || a.Wo.dtype != DT_MXFP4 || a.K % mx8::kBK) return -1;
    if (a.w_tiled && (a.N % 64 || mx8::kBRW != 64)) return -1;
    dim3 grid((unsigned)xcd_grid(ceil_div(a.N, mx8::L::BN) * a.max_tiles));
    if (a.rows_cap < (int64_t)kThinRows * a.E)
      hipLaunchKernelGGL(grouped_down_mx8_kernel<kStream>, grid, dim3(mx8::L::NT), 0, stream, a);
    else
      hipLaunchKernelGGL(grouped_down_mx8_kernel<0>, grid, dim3(mx8::L::NT), 0, stream, a);
    return (int)hipGetLastError();
  }
  if (a.w_tiled) {
    dim3 grid((unsigned)xcd_grid(ceil_div(a.N, bt::BN) * a.max_tiles));
    if (a.Wo.dtype == DT_MXFP4 && a.bm == bt::Thin::BM)
      hipLaunchKernelGGL(grouped_down_btmx_kernel<bt::Thin>, grid, dim3(bt::NW * 64), 0, stream, a);
    else if (a.Wo.dtype == DT_MXFP4 && a.bm == bt::Wide::BM)
      hipLaunchKernelGGL(grouped_down_btmx_kernel<bt::Wide>, grid, dim3(bt::NW * 64), 0, stream, a);
    else if (a.Wo.dtype == DT_BF16 && a.bm == bt::BM)
      hipLaunchKernelGGL(grouped_down_bt_kernel, grid, dim3(bt::NW * 64), 0, stream, a);
    else
      return -1;
    return (int)hipGetLastError();
  }
  if (a.bm == GroupBigCfg::BM && a.bm != GroupCfg::BM) {
    if (a.Wo.dtype != DT_BF16) return -1;
    dim3 grid((unsigned)xcd_grid(ceil_div(a.N, GroupBigCfg::BN) * a.max_tiles));
    hipLaunchKernelGGL(grouped_down_big_kernel, grid, dim3(GroupBigCfg::NT), 0, stream, a);
    return (int)hipGetLastError();
  }
  if (a.bm != GroupCfg::BM) return -1;
  using C = GroupCfg;
  dim3 grid((unsigned)xcd_grid(ceil_div(a.N, C::BN) * a.max_tiles));
  if (a.Wo.dtype == DT_MXFP4) hipLaunchKernelGGL(grouped_down_kernel<true>, grid, dim3(C::NT), 0, stream, a);
  else hipLaunchKernelGGL(grouped_down_kernel<false>, grid, dim3(C::NT), 0, stream, a);
  return (int)hipGetLastError();
}

int launch_decode_mxfp4(const WOperand& w, int64_t rows, int K, void* out, hipStream_t stream) {
  if (w.dtype != DT_MXFP4 || K % 32 || rows < 0) return -1;
  const int64_t blocks = rows * (K / 32);
  if (blocks == 0) return 0;
  const int64_t grid = ceil_div(blocks, 256) < 8192 ? ceil_div(blocks, 256) : 8192;
  hipLaunchKernelGGL(decode_mxfp4_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const uint8_t*)w.data, w.scale, (bf16_t*)out, blocks);
  return (int)hipGetLastError();
}

int launch_multiseg(const MultiSegArgs& a, hipStream_t stream) {
  if (a.act_dtype == DT_F32) return launch_multiseg_f32(a, stream);
  if (a.M == 0) return 0;
  using C = DenseCfg;
  dim3 grid((unsigned)xcd_grid(ceil_div(a.N, C::BN) * ceil_div(a.M, C::BM)));
  // only the last segment (W_up) may be MXFP4, and only in the split form (the
  // single pass takes bf16 weights: an MXFP4 W_up is decoded to bf16 first)
  for (int i = 0; i + 1 < a.nseg; ++i)
    if (a.seg[i].B.dtype == DT_MXFP4) return -1;
  if (multiseg_slices(a.act_dtype, a.M, a.N, a.nseg) > 0) {
    const int e = launch_multiseg_partials(a, 0, a.nseg, stream);
    return e != 0 ? e : launch_multiseg_reduce(a, stream);
  }
  for (int i = 0; i < a.nseg; ++i)
    if (a.seg[i].B.dtype != DT_BF16) return -1;
  hipLaunchKernelGGL(multiseg_kernel, grid, dim3(DenseCfg::NT), 0, stream, a);
  return (int)hipGetLastError();
}

int launch_multiseg_partials(const MultiSegArgs& a, int s0, int ns, hipStream_t stream) {
  if (a.M == 0 || ns == 0) return 0;
  if (multiseg_slices(a.act_dtype, a.M, a.N, a.nseg) == 0 || s0 < 0 || s0 + ns > a.nseg) return -1;
  for (int i = 0; i + 1 < a.nseg; ++i)
    if (a.seg[i].B.dtype == DT_MXFP4) return -1;   // only the last segment may be MXFP4
  const bool last_mx = a.seg[a.nseg - 1].B.dtype == DT_MXFP4;
  using CS = SplitCfg;
  dim3 g2((unsigned)xcd_grid(ceil_div(a.N, CS::BN) * ceil_div(a.M, CS::BM) * ns));
  if (last_mx) hipLaunchKernelGGL(multiseg_split_kernel<true>, g2, dim3(CS::NT), 0, stream, a, s0, ns);
  else hipLaunchKernelGGL(multiseg_split_kernel<false>, g2, dim3(CS::NT), 0, stream, a, s0, ns);
  return (int)hipGetLastError();
}

int launch_multiseg_reduce(const MultiSegArgs& a, hipStream_t stream) {
  if (a.M == 0) return 0;
  if (multiseg_slices(a.act_dtype, a.M, a.N, a.nseg) == 0) return -1;
  const int64_t n4 = (int64_t)a.M * a.N / 4;
  hipLaunchKernelGGL(reduce_store_kernel, dim3(reduce_blocks(n4)), dim3(256), 0, stream, a.P,
                     a.nseg, a.M, a.N, (bf16_t*)a.C, a.ldc);
  return (int)hipGetLastError();
}

// Split K until the grid has about two blocks per CU (small batches).
int router_logit_splits(int T, int E, int d) {
  const int64_t tiles = ceil_div(T, LogitCfg::BM) * ceil_div(E, LogitCfg::BN);
  int splits = 1;
  while (tiles * splits < 512 && d / (splits * 2) >= 4 * LogitCfg::BK) splits *= 2;
  return splits;
}

int launch_router_logits(const LogitsArgs& a, hipStream_t stream) {
  if (a.T == 0) return 0;
  if (a.splits > 1) {
    const int64_t n = (int64_t)a.T * a.E;
    const int64_t blocks = ceil_div(n, 256) < 4096 ? ceil_div(n, 256) : 4096;
    hipLaunchKernelGGL(zero_f32, dim3((unsigned)blocks), dim3(256), 0, stream, a.L, n);
  }
  const int64_t items = ceil_div(a.T, LogitCfg::BM) * ceil_div(a.E, LogitCfg::BN) * a.splits;
  hipLaunchKernelGGL(logits_kernel, dim3((unsigned)xcd_grid(items)), dim3(LogitCfg::NT), 0, stream, a);
  return (int)hipGetLastError();
}

}  // namespace moe
