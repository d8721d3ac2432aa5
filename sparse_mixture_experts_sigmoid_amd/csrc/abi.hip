// C ABI of the Stable LatentMoE layer (declared in include/moe.h): host-side
// validation, workspace planning and the launch sequence. All validation runs
// before any HIP call, so every error path is testable without a GPU.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(int hip_status, const char* where) {
  if (hip_status == -1) return fail(MOE_ERR_UNSUPPORTED, "%s: no kernel for this configuration", where);
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString((hipError_t)hip_status));
}

#define MOE_LAUNCH(call, where)                  \
  do {                                           \
    int st_ = (call);                            \
    if (st_ != 0) return hip_fail(st_, where);   \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elem_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

constexpr int kMaxExperts = 4096;

int check_desc(const moe_desc_t* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
  if (d->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d < 0", d->T);
  if (d->d_model <= 0 || d->d_latent <= 0 || d->d_ff <= 0)
    return fail(MOE_ERR_INVALID_ARG, "d_model, d_latent and d_ff must be > 0");
  if (d->n_shared < 0) return fail(MOE_ERR_INVALID_ARG, "n_shared < 0");
  if (d->n_shared > 0 && d->d_ff_shared <= 0)
    return fail(MOE_ERR_INVALID_ARG, "d_ff_shared must be > 0 when n_shared > 0");
  if (d->n_experts <= 0) return fail(MOE_ERR_INVALID_ARG, "n_experts must be > 0");
  if (d->top_k < 1 || d->top_k > d->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k = %d must be in [1, n_experts = %d]", d->top_k,
                d->n_experts);
  if (!(d->situ_c > 0.0f) || !std::isfinite(d->situ_c))
    return fail(MOE_ERR_INVALID_ARG, "situ_c must be finite and > 0");
  if (!(d->rms_eps >= 0.0f) || !std::isfinite(d->rms_eps))
    return fail(MOE_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  const int dts[4] = {d->act_dtype, d->expert_w_dtype, d->latent_w_dtype, d->dense_w_dtype};
  for (int v : dts)
    if (v != MOE_F32 && v != MOE_BF16 && v != MOE_MXFP4)
      return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", v);
  if (d->act_dtype == MOE_F32) {
    if (d->expert_w_dtype != MOE_F32 || d->latent_w_dtype != MOE_F32 || d->dense_w_dtype != MOE_F32)
      return fail(MOE_ERR_UNSUPPORTED, "fp32 activations need fp32 weights");
  } else if (d->act_dtype == MOE_BF16) {
    if (d->dense_w_dtype != MOE_BF16)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 activations need bf16 router/shared weights");
    if (d->expert_w_dtype == MOE_F32 || d->latent_w_dtype == MOE_F32)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 activations need bf16 or MXFP4 expert/latent weights");
  } else {
    return fail(MOE_ERR_UNSUPPORTED, "activations must be fp32 or bf16");
  }
  if (d->d_model % 32 || d->d_latent % 32 || d->d_ff % 32 ||
      (d->n_shared > 0 && d->d_ff_shared % 32))
    return fail(MOE_ERR_UNSUPPORTED, "d_model, d_latent, d_ff, d_ff_shared must be multiples of 32");
  if (d->expert_act_mxfp8 != 0 && d->expert_act_mxfp8 != 1)
    return fail(MOE_ERR_INVALID_ARG, "expert_act_mxfp8 must be 0 or 1");
  if (d->expert_act_mxfp8 &&
      (d->act_dtype != MOE_BF16 || d->expert_w_dtype != MOE_MXFP4 || d->d_latent % 128 || d->d_ff % 128))
    return fail(MOE_ERR_UNSUPPORTED, "MXFP8 expert activations need bf16 activations, MXFP4 expert "
                "weights and d_latent, d_ff multiples of 128");
  if (d->expert_w_tiled != 0 && d->expert_w_tiled != 1)
    return fail(MOE_ERR_INVALID_ARG, "expert_w_tiled must be 0 or 1");
  if (d->expert_w_tiled && d->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "tiled expert weights need bf16 activations");
  if (d->n_experts > kMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", kMaxExperts);
  if (d->n_shared + 1 > moe::kMaxSegments)
    return fail(MOE_ERR_UNSUPPORTED, "n_shared > %d", moe::kMaxSegments - 1);
  const int64_t rows = (int64_t)d->T * d->top_k;
  if (rows > (int64_t)1 << 30) return fail(MOE_ERR_UNSUPPORTED, "T * top_k too large");
  if (rows / 128 + d->n_experts > 65535 || (int64_t)d->T / 128 + 1 > 65535)
    return fail(MOE_ERR_UNSUPPORTED, "batch too large for one launch");
  // the routed experts gather their z rows through one buffer resource with
  // 32-bit offsets: the whole z must stay under 2 GiB
  if (d->act_dtype == MOE_BF16 && (int64_t)d->T * d->d_latent * 2 >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T * d_latent * 2 bytes of z must stay under 2 GiB (T = %d)", d->T);
  return MOE_OK;
}

// ------------------------------------------------------------------------------------------
// workspace planning
// ------------------------------------------------------------------------------------------

struct Plan {
  size_t total = 0;
  size_t take(size_t bytes) {
    size_t off = total;
    total += (bytes + 255) & ~(size_t)255;
    return off;
  }
};

struct LayerWs {
  size_t s, key, norms, idx, gate, counts, offsets, perm, inv, blk, z, tile_off, tile_info, H, O, n, Hs, P;
  size_t zq, zqs, hq, hqs;   // MXFP8 z and h (codes, scales) of the scaled-MFMA expert path
  size_t wld, wlu;           // bf16 copies of MXFP4 W_ld / W_lu for the single-pass dense GEMMs
};

int max_tiles(const moe_desc_t* d) {
  const int bm = moe::grouped_bm(d->act_dtype, d->expert_w_dtype, d->expert_act_mxfp8, d->expert_w_tiled, (int64_t)d->T * d->top_k, d->n_experts);
  return (int)(((int64_t)d->T * d->top_k + bm - 1) / bm + d->n_experts);
}

void plan_route(const moe_desc_t* d, Plan& p, LayerWs& w) {
  w.s = p.take((size_t)d->T * d->n_experts * 4);
  w.key = p.take((size_t)d->T * d->n_experts * 4);
  w.norms = p.take((size_t)(d->T + d->n_experts) * 4);
}
void plan_permute(const moe_desc_t* d, Plan& p, LayerWs& w) {
  w.blk = p.take((size_t)moe::permute_blocks(d->T) * d->n_experts * 4);
}
// tile table and, on the scaled-MFMA path, the MXFP8 copy of z
void plan_gate_up(const moe_desc_t* d, Plan& p, LayerWs& w) {
  w.tile_off = p.take((size_t)(d->n_experts + 1) * 4);
  w.tile_info = p.take((size_t)max_tiles(d) * 16);
  if (d->expert_act_mxfp8) {
    w.zq = p.take((size_t)d->T * d->d_latent);
    w.zqs = p.take((size_t)d->T * d->d_latent / 32);
  }
}
void plan_expert(const moe_desc_t* d, Plan& p, LayerWs& w) {
  plan_gate_up(d, p, w);
  // bf16 h [T k, F]; the scaled-MFMA path writes h only in MXFP8 (hq, hqs)
  w.H = p.take(d->expert_act_mxfp8 ? 0 : (size_t)d->T * d->top_k * d->d_ff * elem_bytes(d->act_dtype));
  if (d->expert_act_mxfp8) {
    const size_t rows = (size_t)d->T * d->top_k;
    w.hq = p.take(rows * d->d_ff);
    w.hqs = p.take(rows * d->d_ff / 32);
  }
}
// fp32 split-K partials of the dense GEMMs that run with few tokens
moe::SplitK latent_split(const moe_desc_t* d) {
  return moe::plan_split(d->act_dtype, d->T, d->d_latent, d->d_model);
}
moe::SplitK shared_split(const moe_desc_t* d) {
  return moe::plan_split(d->act_dtype, d->T, 2 * d->n_shared * d->d_ff_shared, d->d_model);
}
size_t latent_partial_bytes(const moe_desc_t* d) {
  return (size_t)latent_split(d).partial_bytes(d->T, d->d_latent);
}
size_t output_partial_bytes(const moe_desc_t* d) {
  const size_t glu = d->n_shared > 0
      ? (size_t)shared_split(d).partial_bytes(d->T, 2 * (int64_t)d->n_shared * d->d_ff_shared) : 0;
  const size_t out = (size_t)moe::multiseg_slices(d->act_dtype, d->T, d->d_model, d->n_shared + 1) *
                     d->T * d->d_model * 4;
  return glu > out ? glu : out;
}
// MXFP4 latent maps at batch sizes where their dense GEMM runs in one pass:
// the weight is decoded once per call (exactly) into a bf16 copy of d_lat x d
// elements in the workspace, and the bf16 GEMM reads that copy. (The split
// form at small batches reads the MXFP4 weight itself.)
bool latent_down_decoded(const moe_desc_t* d) {
  return d->latent_w_dtype == MOE_MXFP4 && d->T > 0 && latent_split(d).splits == 0;
}
bool output_decoded(const moe_desc_t* d) {
  return d->latent_w_dtype == MOE_MXFP4 && d->T > 0 &&
         moe::multiseg_slices(d->act_dtype, d->T, d->d_model, d->n_shared + 1) == 0;
}
size_t latent_copy_bytes(const moe_desc_t* d) { return (size_t)d->d_latent * d->d_model * 2; }

void plan_latent(const moe_desc_t* d, Plan& p, LayerWs& w) {
  w.P = p.take(latent_partial_bytes(d));
  w.wld = p.take(latent_down_decoded(d) ? latent_copy_bytes(d) : 0);
}
void plan_output(const moe_desc_t* d, Plan& p, LayerWs& w) {
  w.Hs = p.take((size_t)d->T * d->n_shared * d->d_ff_shared * elem_bytes(d->act_dtype));
  w.P = p.take(output_partial_bytes(d));
  w.wlu = p.take(output_decoded(d) ? latent_copy_bytes(d) : 0);
}

Plan plan_layer(const moe_desc_t* d, LayerWs& w) {
  Plan p;
  plan_route(d, p, w);
  const size_t tk = (size_t)d->T * d->top_k;
  w.idx = p.take(tk * 4);
  w.gate = p.take(tk * 4);
  w.counts = p.take((size_t)d->n_experts * 4);
  w.offsets = p.take((size_t)(d->n_experts + 1) * 4);
  w.perm = p.take(tk * 4);
  w.inv = p.take(tk * 4);
  plan_permute(d, p, w);
  w.z = p.take((size_t)d->T * d->d_latent * elem_bytes(d->act_dtype));
  plan_expert(d, p, w);
  w.O = p.take(tk * d->d_latent * elem_bytes(d->act_dtype));
  w.n = p.take((size_t)d->T * d->d_latent * elem_bytes(d->act_dtype));
  w.Hs = p.take((size_t)d->T * d->n_shared * d->d_ff_shared * elem_bytes(d->act_dtype));
  // one partial buffer serves latent down, shared gate/up and the output GEMM (in turn)
  const size_t lp = latent_partial_bytes(d), op = output_partial_bytes(d);
  w.P = p.take(lp > op ? lp : op);
  w.wld = p.take(latent_down_decoded(d) ? latent_copy_bytes(d) : 0);
  w.wlu = p.take(output_decoded(d) ? latent_copy_bytes(d) : 0);
  return p;
}

size_t ws_bytes_for(const moe_desc_t* d, int op) {
  Plan p;
  LayerWs w{};
  switch (op) {
    case MOE_OP_ROUTE: plan_route(d, p, w); break;
    case MOE_OP_PERMUTE: plan_permute(d, p, w); break;
    case MOE_OP_LATENT_DOWN: plan_latent(d, p, w); break;
    case MOE_OP_EXPERT_FFN: plan_expert(d, p, w); break;
    case MOE_OP_EXPERT_GATE_UP: plan_gate_up(d, p, w); break;
    case MOE_OP_COMBINE: break;
    case MOE_OP_OUTPUT: plan_output(d, p, w); break;
    case MOE_OP_LAYER: p = plan_layer(d, w); break;
    default: return 0;
  }
  return p.total;
}

int check_ws(const moe_desc_t* d, int op, void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(d, op);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  if (need > 0 && (ws == nullptr || !aligned16(ws)))
    return fail(MOE_ERR_INVALID_ARG, "workspace is NULL or not 16-byte aligned");
  return MOE_OK;
}

int need_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

// A buffer whose size scales with T: may be NULL for an empty batch.
int need_ptr_t(const moe_desc_t* d, const void* p, const char* name) {
  if (d->T == 0 && p == nullptr) return MOE_OK;
  return need_ptr(p, name);
}

int opt_ptr(const void* p, const char* name) {
  if (p != nullptr && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

int need_w(const moe_w_t& w, int dtype, const char* name) {
  if (int st = need_ptr(w.data, name)) return st;
  if (dtype == MOE_MXFP4 && w.scale == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "%s: MXFP4 weight without scales", name);
  if (dtype == MOE_MXFP4 && (uintptr_t)w.scale % 4)
    return fail(MOE_ERR_INVALID_ARG, "%s: MXFP4 scales are not 4-byte aligned", name);
  return MOE_OK;
}

#define MOE_CHECK(expr)           \
  do {                            \
    int st_ = (expr);             \
    if (st_ != MOE_OK) return st_; \
  } while (0)

moe::WOperand wop(const moe_w_t& w, int dtype) { return moe::WOperand{w.data, w.scale, dtype}; }

char* at(void* ws, size_t off) { return (char*)ws + off; }

// ------------------------------------------------------------------------------------------
// stage tracing: per traced call and stage, a start and an end event recorded on the stream
// the stage runs on
// ------------------------------------------------------------------------------------------

const char* const kStageNames[MOE_TRACE_STAGES] = {
    "router", "topk", "permute", "latent_down", "tile_table",
    "expert_gate_up", "expert_down", "combine", "shared_gate_up", "output"};

constexpr uint32_t kAllStages = (1u << MOE_TRACE_STAGES) - 1;

struct Trace {
  std::mutex mu;
  int max_calls = 0;
  int used = 0;
  uint32_t mask = kAllStages;  // stages whose events are recorded
  std::vector<hipEvent_t> ev;  // max_calls * 2 * MOE_TRACE_STAGES
};
Trace g_trace;

struct Marker;
// A slot for one traced call (slot -1: not traced) and the stages it records.
Marker trace_begin();

constexpr size_t kTraceEvents = 2 * MOE_TRACE_STAGES;   // per traced call

// Stage markers of a traced call. Tracing never fails the layer: an event that
// could not be recorded leaves that stage's time unreadable (moe_trace_read
// then returns the HIP error).
struct Marker {
  int slot;
  uint32_t mask = 0;
  bool on(int stage) const { return slot >= 0 && ((mask >> stage) & 1u); }
  void beg(int stage, hipStream_t s) const {
    if (on(stage)) (void)hipEventRecord(g_trace.ev[(size_t)slot * kTraceEvents + 2 * stage], s);
  }
  void end(int stage, hipStream_t s) const {
    if (on(stage)) (void)hipEventRecord(g_trace.ev[(size_t)slot * kTraceEvents + 2 * stage + 1], s);
  }
};

Marker trace_begin() {
  std::lock_guard<std::mutex> lk(g_trace.mu);
  if (g_trace.used >= g_trace.max_calls) return Marker{-1, 0};
  return Marker{g_trace.used++, g_trace.mask};
}

// ------------------------------------------------------------------------------------------
// stages (arguments already validated)
// ------------------------------------------------------------------------------------------

// bf16 x and W_r without a request for all scores: matrix-core logits, then
// the exact fixed-order recheck of the near-boundary experts only (same result
// bit for bit). Otherwise every (token, expert) logit in fixed order on VALU.
int do_route(const moe_desc_t* d, const void* x, moe_w_t router, const float* bias, int32_t* idx,
             float* gate, float* s, float* key, float* norms, bool want_scores, hipStream_t st,
             Marker mk = {-1}) {
  if (!want_scores && d->act_dtype == MOE_BF16 && d->dense_w_dtype == MOE_BF16 &&
      moe::router_select_supported(d->n_experts, d->d_model)) {
    float* xn = norms;
    float* wn = norms + d->T;
    mk.beg(0, st);
    MOE_LAUNCH(moe::launch_row_norms(x, d->T, d->d_model, xn, st), "row_norms");
    MOE_LAUNCH(moe::launch_row_norms(router.data, d->n_experts, d->d_model, wn, st), "row_norms");
    moe::LogitsArgs la{x, router.data, d->T, d->n_experts, d->d_model,
                       moe::router_logit_splits(d->T, d->n_experts, d->d_model), s};
    MOE_LAUNCH(moe::launch_router_logits(la, st), "router_logits");
    mk.end(0, st);
    mk.beg(1, st);
    moe::SelectArgs sa{s, x, router.data, bias, xn, wn, d->T, d->n_experts, d->d_model,
                       d->top_k, idx, gate};
    MOE_LAUNCH(moe::launch_router_select(sa, st), "router_select");
    mk.end(1, st);
    return MOE_OK;
  }
  moe::RouterArgs ra{x, d->act_dtype, router.data, d->dense_w_dtype, bias, d->T, d->d_model,
                     d->n_experts, s, key};
  mk.beg(0, st);
  MOE_LAUNCH(moe::launch_router(ra, st), "router");
  mk.end(0, st);
  mk.beg(1, st);
  moe::TopkArgs ta{s, key, d->T, d->n_experts, d->top_k, idx, gate};
  MOE_LAUNCH(moe::launch_topk(ta, st), "topk");
  mk.end(1, st);
  return MOE_OK;
}

int do_permute(const moe_desc_t* d, const int32_t* idx, int32_t* counts, int32_t* offsets,
               int32_t* perm, int32_t* inv, int32_t* blk, hipStream_t st) {
  moe::PermuteArgs pa{idx, d->T, d->n_experts, d->top_k, counts, offsets, perm, inv, blk};
  MOE_LAUNCH(moe::launch_permute(pa, st), "permute");
  return MOE_OK;
}

// wcopy: workspace for the bf16 copy of an MXFP4 W_ld (used when
// latent_down_decoded)
int do_latent_down(const moe_desc_t* d, const void* x, moe_w_t w, void* z, float* P, void* wcopy,
                   hipStream_t st) {
  moe::WOperand W = wop(w, d->latent_w_dtype);
  if (latent_down_decoded(d)) {
    MOE_LAUNCH(moe::launch_decode_mxfp4(W, d->d_latent, d->d_model, wcopy, st), "latent_down (decode)");
    W = moe::WOperand{wcopy, nullptr, MOE_BF16};
  }
  moe::DenseArgs a{x, d->d_model, W, d->T, d->d_latent, d->d_model, z,
                   d->d_latent, d->act_dtype, latent_split(d), P};
  MOE_LAUNCH(moe::launch_dense(a, st), "latent_down");
  return MOE_OK;
}

// MXFP8 copies of z and h for the scaled-MFMA expert path (workspace)
struct MxBufs {
  uint8_t *zq = nullptr, *zqs = nullptr, *hq = nullptr, *hqs = nullptr;
};
MxBufs mx_bufs(const moe_desc_t* d, void* ws, const LayerWs& lw) {
  MxBufs m;
  if (d->expert_act_mxfp8) {
    m.zq = (uint8_t*)at(ws, lw.zq);
    m.zqs = (uint8_t*)at(ws, lw.zqs);
    m.hq = (uint8_t*)at(ws, lw.hq);
    m.hqs = (uint8_t*)at(ws, lw.hqs);
  }
  return m;
}

// Tile table, then h = act(W_g z, W_v z) for every permuted row: into H (act
// dtype) when H is set, else (scaled-MFMA path only) straight into MXFP8 codes
// hq and scales hqs, the down GEMM's input.
int do_gate_up(const moe_desc_t* d, const void* z, const int32_t* perm, const int32_t* offsets,
               const moe_weights_t* w, int32_t* tile_off, int32_t* tile_info, void* H,
               const MxBufs& mx, hipStream_t st, Marker mk = {-1}) {
  const bool q8 = d->expert_act_mxfp8 != 0;
  const int bm = moe::grouped_bm(d->act_dtype, d->expert_w_dtype, d->expert_act_mxfp8, d->expert_w_tiled, (int64_t)d->T * d->top_k, d->n_experts);
  mk.beg(4, st);
  if (d->T > 0)
    MOE_LAUNCH(moe::launch_tile_table(offsets, d->n_experts, bm, tile_off, tile_info, st),
               "tile_table");
  mk.end(4, st);
  mk.beg(5, st);
  if (q8 && d->T > 0)
    MOE_LAUNCH(moe::launch_quantize_mx8(z, d->T, d->d_latent, d->d_latent, mx.zq, mx.zqs, st),
               "quantize_z");
  moe::GroupedGluArgs g{};
  g.Z = q8 ? (const void*)mx.zq : z; g.ldz = d->d_latent; g.T = d->T; g.rows_cap = d->T * d->top_k;
  g.act_mx8 = q8; g.z_scale = mx.zqs; g.w_tiled = d->expert_w_tiled;
  g.hq = H == nullptr ? mx.hq : nullptr; g.hqs = H == nullptr ? mx.hqs : nullptr;
  g.perm_src = perm; g.topk = d->top_k; g.offsets = offsets; g.tile_off = tile_off;
  g.tile_info = tile_info;
  g.max_tiles = max_tiles(d);
  g.Wg = wop(w->exp_gate, d->expert_w_dtype);
  g.Wv = wop(w->exp_up, d->expert_w_dtype);
  g.E = d->n_experts; g.F = d->d_ff; g.K = d->d_latent;
  g.H = H; g.c = d->situ_c; g.act_dtype = d->act_dtype; g.bm = bm;
  if (d->T > 0) MOE_LAUNCH(moe::launch_grouped_glu(g, st), "expert_gate_up");
  mk.end(5, st);
  return MOE_OK;
}

int do_experts(const moe_desc_t* d, const void* z, const int32_t* perm, const int32_t* offsets,
               const moe_weights_t* w, void* o_perm, int32_t* tile_off, int32_t* tile_info, void* H,
               const MxBufs& mx, hipStream_t st, Marker mk = {-1}) {
  const bool q8 = d->expert_act_mxfp8 != 0;
  const int bm = moe::grouped_bm(d->act_dtype, d->expert_w_dtype, d->expert_act_mxfp8, d->expert_w_tiled, (int64_t)d->T * d->top_k, d->n_experts);
  const int mt = max_tiles(d);
  const int rows_cap = d->T * d->top_k;
  // the scaled-MFMA path writes h straight in MXFP8 (the down GEMM's input)
  MOE_CHECK(do_gate_up(d, z, perm, offsets, w, tile_off, tile_info, q8 ? nullptr : H, mx, st, mk));
  mk.beg(6, st);
  moe::GroupedDownArgs dn{};
  dn.H = q8 ? (const void*)mx.hq : H; dn.ldh = d->d_ff; dn.rows_cap = rows_cap;
  dn.act_mx8 = q8; dn.h_scale = mx.hqs; dn.w_tiled = d->expert_w_tiled;
  dn.offsets = offsets; dn.tile_off = tile_off; dn.tile_info = tile_info; dn.max_tiles = mt;
  dn.Wo = wop(w->exp_down, d->expert_w_dtype);
  dn.E = d->n_experts; dn.N = d->d_latent; dn.K = d->d_ff;
  dn.O = o_perm; dn.act_dtype = d->act_dtype; dn.bm = bm;
  if (d->T > 0) MOE_LAUNCH(moe::launch_grouped_down(dn, st), "expert_down");
  mk.end(6, st);
  return MOE_OK;
}

int do_combine(const moe_desc_t* d, const void* o_perm, const int32_t* inv, const float* gate,
               const float* gain, void* n, float* u, hipStream_t st) {
  moe::CombineArgs c{o_perm, inv, gate, gain, d->T, d->top_k, d->d_latent, d->rms_eps,
                     n, d->d_latent, u, d->act_dtype};
  MOE_LAUNCH(moe::launch_combine(c, st), "combine");
  return MOE_OK;
}

// Shared experts' gate/up + SiTU-GLU: Hs = act(x W_g^s^T, x W_v^s^T), all S at once.
int do_shared_glu(const moe_desc_t* d, const void* x, const moe_weights_t* w, void* Hs, float* P,
                  hipStream_t st, Marker mk = {-1}) {
  const int S = d->n_shared, Fs = d->d_ff_shared, D = d->d_model;
  mk.beg(8, st);
  if (S == 0) {
    mk.end(8, st);
    return MOE_OK;
  }
  moe::GluArgs g{};
  g.A = x; g.lda = D;
  g.Wg = wop(w->sh_gate, d->dense_w_dtype);
  g.Wv = wop(w->sh_up, d->dense_w_dtype);
  g.M = d->T; g.F = S * Fs; g.K = D;
  g.H = Hs; g.ldh = (int64_t)S * Fs; g.c = d->situ_c; g.act_dtype = d->act_dtype;
  g.split = shared_split(d); g.P = P;
  MOE_LAUNCH(moe::launch_glu(g, st), "shared_gate_up");
  mk.end(8, st);
  return MOE_OK;
}

// y = sum_s Hs_s W_o^s^T + n W_up^T: one GEMM whose K runs over the shared
// experts' down projections and then W_up.
// The output GEMM: y = sum_s Hs_s W_os_s^T + n W_lu^T as one GEMM over the
// concatenated K segments (shared experts first, W_up last).
moe::MultiSegArgs output_args(const moe_desc_t* d, const void* n, const moe_weights_t* w, void* y,
                              const void* Hs, float* P) {
  const int S = d->n_shared, Fs = d->d_ff_shared, D = d->d_model;
  const size_t eb = elem_bytes(d->act_dtype);
  moe::MultiSegArgs m{};
  for (int s = 0; s < S; ++s) {
    m.seg[s].A = (const char*)Hs + (size_t)s * Fs * eb;
    m.seg[s].lda = (int64_t)S * Fs;
    m.seg[s].B = moe::WOperand{(const char*)w->sh_down.data + (size_t)s * D * Fs * eb, nullptr,
                               d->dense_w_dtype};
    m.seg[s].K = Fs;
  }
  m.seg[S].A = n;
  m.seg[S].lda = d->d_latent;
  m.seg[S].B = wop(w->lat_up, d->latent_w_dtype);
  m.seg[S].K = d->d_latent;
  m.nseg = S + 1;
  m.M = d->T; m.N = D; m.C = y; m.ldc = D; m.act_dtype = d->act_dtype; m.P = P;
  return m;
}

// wcopy: workspace for the bf16 copy of an MXFP4 W_up (used when output_decoded)
int do_output_gemm(const moe_desc_t* d, const void* n, const moe_weights_t* w, void* y,
                   const void* Hs, float* P, void* wcopy, hipStream_t st, Marker mk = {-1}) {
  mk.beg(9, st);
  moe::MultiSegArgs m = output_args(d, n, w, y, Hs, P);
  if (output_decoded(d)) {
    moe::Segment& last = m.seg[m.nseg - 1];
    MOE_LAUNCH(moe::launch_decode_mxfp4(last.B, d->d_model, d->d_latent, wcopy, st), "output (decode)");
    last.B = moe::WOperand{wcopy, nullptr, MOE_BF16};
  }
  MOE_LAUNCH(moe::launch_multiseg(m, st), "output");
  mk.end(9, st);
  return MOE_OK;
}

// Whether the output GEMM takes its split form (per-segment fp32 partials and
// an ordered sum): then the shared experts' partials need only Hs and can be
// made early, off the critical path.
bool output_split(const moe_desc_t* d) {
  return d->n_shared > 0 &&
         moe::multiseg_slices(d->act_dtype, d->T, d->d_model, d->n_shared + 1) > 0;
}

int do_output(const moe_desc_t* d, const void* x, const void* n, const moe_weights_t* w, void* y,
              void* Hs, float* P, void* wcopy, hipStream_t st) {
  MOE_CHECK(do_shared_glu(d, x, w, Hs, P, st));
  return do_output_gemm(d, n, w, y, Hs, P, wcopy, st);
}

// A second stream per device for the work of moe_layer_forward that does not
// depend on the routing (latent down, shared experts' gate/up): forked from
// and joined back into the caller's stream with events, so the caller sees one
// stream-ordered call. Created on first use (default priority), kept for the
// life of the process; `mu` serialises the fork / join of concurrent callers.
struct SideStream {
  std::mutex mu;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, join_out = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::mutex g_side_init;

int side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail((int)e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_side_init);
  SideStream& sd = g_side[dev];
  if (sd.s == nullptr) {
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr, jo = nullptr;
    e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&jo, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (jo) (void)hipEventDestroy(jo);
      if (j) (void)hipEventDestroy(j);
      if (f) (void)hipEventDestroy(f);
      if (s) (void)hipStreamDestroy(s);
      return hip_fail((int)e, "side stream");
    }
    sd.fork = f;
    sd.join = j;
    sd.join_out = jo;
    sd.s = s;
  }
  *out = &sd;
  return MOE_OK;
}

int check_layer_args(const moe_desc_t* d, const moe_weights_t* w, const void* x, const void* y,
                     const int32_t* topk_idx_opt, const float* topk_gate_opt, const int32_t* counts_opt) {
  MOE_CHECK(check_desc(d));
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  MOE_CHECK(need_ptr_t(d, x, "x"));
  MOE_CHECK(need_ptr_t(d, y, "y"));
  MOE_CHECK(need_w(w->router, d->dense_w_dtype, "router"));
  MOE_CHECK(need_ptr(w->router_bias, "router_bias"));
  MOE_CHECK(need_w(w->lat_down, d->latent_w_dtype, "lat_down"));
  MOE_CHECK(need_w(w->lat_up, d->latent_w_dtype, "lat_up"));
  MOE_CHECK(opt_ptr(w->rms_gain, "rms_gain"));
  MOE_CHECK(need_w(w->exp_gate, d->expert_w_dtype, "exp_gate"));
  MOE_CHECK(need_w(w->exp_up, d->expert_w_dtype, "exp_up"));
  MOE_CHECK(need_w(w->exp_down, d->expert_w_dtype, "exp_down"));
  if (d->n_shared > 0) {
    MOE_CHECK(need_w(w->sh_gate, d->dense_w_dtype, "sh_gate"));
    MOE_CHECK(need_w(w->sh_up, d->dense_w_dtype, "sh_up"));
    MOE_CHECK(need_w(w->sh_down, d->dense_w_dtype, "sh_down"));
  }
  MOE_CHECK(opt_ptr(topk_idx_opt, "topk_idx"));
  MOE_CHECK(opt_ptr(topk_gate_opt, "topk_gate"));
  MOE_CHECK(opt_ptr(counts_opt, "counts"));
  return MOE_OK;
}

// The layer on workspace ws. With a side stream sd (held locked by the caller)
// the routing-independent GEMMs (latent down, shared gate/up) run on it,
// forked from and joined back into st; without one everything runs on st in
// order.
int run_layer(const moe_desc_t* d, const moe_weights_t* w, const void* x, void* y, int32_t* topk_idx_opt,
              float* topk_gate_opt, int32_t* counts_opt, void* ws, hipStream_t st, SideStream* sd,
              Marker mk) {
  LayerWs lw{};
  plan_layer(d, lw);
  int32_t* idx = topk_idx_opt ? topk_idx_opt : (int32_t*)at(ws, lw.idx);
  float* gate = topk_gate_opt ? topk_gate_opt : (float*)at(ws, lw.gate);
  int32_t* counts = counts_opt ? counts_opt : (int32_t*)at(ws, lw.counts);
  int32_t* offsets = (int32_t*)at(ws, lw.offsets);
  int32_t* perm = (int32_t*)at(ws, lw.perm);
  int32_t* inv = (int32_t*)at(ws, lw.inv);
  hipStream_t side = st;
  if (sd != nullptr) {
    MOE_LAUNCH((int)hipEventRecord(sd->fork, st), "fork");
    MOE_LAUNCH((int)hipStreamWaitEvent(sd->s, sd->fork, 0), "fork");
    side = sd->s;
  }
  // the routing-independent GEMMs (z and the shared experts' H)
  mk.beg(3, side);
  MOE_CHECK(do_latent_down(d, x, w->lat_down, at(ws, lw.z), (float*)at(ws, lw.P), at(ws, lw.wld), side));
  mk.end(3, side);
  MOE_CHECK(do_shared_glu(d, x, w, at(ws, lw.Hs), (float*)at(ws, lw.P), side, mk));
  if (sd != nullptr) MOE_LAUNCH((int)hipEventRecord(sd->join, sd->s), "join");
  // split output GEMM: the shared experts' partials right after their H, on
  // the side stream, while the routed experts run (same slices, same ordered
  // sum at the end: the same bits as making them after the combine)
  const moe::MultiSegArgs out = output_args(d, at(ws, lw.n), w, y, at(ws, lw.Hs), (float*)at(ws, lw.P));
  const bool early = sd != nullptr && output_split(d);
  if (early) {
    MOE_LAUNCH(moe::launch_multiseg_partials(out, 0, d->n_shared, sd->s), "output (shared partials)");
    MOE_LAUNCH((int)hipEventRecord(sd->join_out, sd->s), "join");
  }
  // routing and permutation, then (after the join) the experts
  MOE_CHECK(do_route(d, x, w->router, w->router_bias, idx, gate, (float*)at(ws, lw.s),
                     (float*)at(ws, lw.key), (float*)at(ws, lw.norms), false, st, mk));
  mk.beg(2, st);
  MOE_CHECK(do_permute(d, idx, counts, offsets, perm, inv, (int32_t*)at(ws, lw.blk), st));
  mk.end(2, st);
  if (sd != nullptr) MOE_LAUNCH((int)hipStreamWaitEvent(st, sd->join, 0), "join");
  MOE_CHECK(do_experts(d, at(ws, lw.z), perm, offsets, w, at(ws, lw.O), (int32_t*)at(ws, lw.tile_off),
                       (int32_t*)at(ws, lw.tile_info), at(ws, lw.H), mx_bufs(d, ws, lw), st, mk));
  mk.beg(7, st);
  MOE_CHECK(do_combine(d, at(ws, lw.O), inv, gate, w->rms_gain, at(ws, lw.n), nullptr, st));
  mk.end(7, st);
  if (early) {
    mk.beg(9, st);
    MOE_LAUNCH(moe::launch_multiseg_partials(out, d->n_shared, 1, st), "output");
    MOE_LAUNCH((int)hipStreamWaitEvent(st, sd->join_out, 0), "join");
    MOE_LAUNCH(moe::launch_multiseg_reduce(out, st), "output");
    mk.end(9, st);
    return MOE_OK;
  }
  MOE_CHECK(do_output_gemm(d, at(ws, lw.n), w, y, at(ws, lw.Hs), (float*)at(ws, lw.P), at(ws, lw.wlu), st,
                           mk));
  return MOE_OK;
}

// Scratch of moe_layer_forward_noalloc, for callers that cannot allocate
// device memory: a fixed array in the code object, one copy on every GPU the
// library runs on, held until the process ends. In host code `scratch` names
// a host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device (with that device current), and only
// that address is ever passed to a kernel. Calls on one GPU share its copy
// (the last call's contents stay); no kernel reads scratch that the same call
// has not written first, so nothing needs clearing between calls. Calls that
// overlap on one GPU race on it.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail((int)e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail((int)e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

// ------------------------------------------------------------------------------------------
// exported entry points
// ------------------------------------------------------------------------------------------

extern "C" {

int moe_check_desc(const moe_desc_t* desc) {
  g_last_error.clear();
  return check_desc(desc);
}

size_t moe_workspace_bytes(const moe_desc_t* desc, int op) {
  if (check_desc(desc) != MOE_OK) return 0;
  return ws_bytes_for(desc, op);
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_trace_stage_name(int stage) {
  return (stage >= 0 && stage < MOE_TRACE_STAGES) ? kStageNames[stage] : "";
}

int moe_trace_enable(int max_calls) { return moe_trace_enable_stages(max_calls, kAllStages); }

int moe_trace_enable_stages(int max_calls, unsigned stage_mask) {
  g_last_error.clear();
  if (max_calls < 0 || max_calls > 100000) return fail(MOE_ERR_INVALID_ARG, "max_calls out of range");
  if (stage_mask & ~kAllStages) return fail(MOE_ERR_INVALID_ARG, "stage_mask has bits past stage %d", MOE_TRACE_STAGES - 1);
  std::lock_guard<std::mutex> lk(g_trace.mu);
  g_trace.mask = stage_mask;
  for (hipEvent_t e : g_trace.ev) hipEventDestroy(e);
  g_trace.ev.clear();
  g_trace.max_calls = 0;
  g_trace.used = 0;
  const size_t n = (size_t)max_calls * kTraceEvents;
  g_trace.ev.resize(n);
  for (size_t i = 0; i < n; ++i) {
    hipError_t e = hipEventCreate(&g_trace.ev[i]);
    if (e != hipSuccess) {
      g_trace.ev.resize(i);
      return hip_fail((int)e, "trace_enable");
    }
  }
  g_trace.max_calls = max_calls;
  return MOE_OK;
}

int moe_trace_read(float* ms, int max_stages, int* ncalls) {
  g_last_error.clear();
  if (ms == nullptr && max_stages > 0) return fail(MOE_ERR_INVALID_ARG, "ms is NULL");
  std::lock_guard<std::mutex> lk(g_trace.mu);
  const int used = g_trace.used;
  const int ns = max_stages < MOE_TRACE_STAGES ? max_stages : MOE_TRACE_STAGES;
  for (int i = 0; i < ns; ++i) ms[i] = ((g_trace.mask >> i) & 1u) ? 0.0f : -1.0f;
  for (int c = 0; c < used; ++c) {
    hipEvent_t* ev = &g_trace.ev[(size_t)c * kTraceEvents];
    for (int i = 0; i < ns; ++i) {
      if (!((g_trace.mask >> i) & 1u)) continue;
      hipError_t e = hipEventSynchronize(ev[2 * i + 1]);
      if (e != hipSuccess) return hip_fail((int)e, "trace_read");
      float t = 0.0f;
      e = hipEventElapsedTime(&t, ev[2 * i], ev[2 * i + 1]);
      if (e != hipSuccess) return hip_fail((int)e, "trace_read");
      ms[i] += t / (float)used;
    }
  }
  if (ncalls) *ncalls = used;
  g_trace.used = 0;
  return MOE_OK;
}

int moe_route(const moe_desc_t* d, const void* x, moe_w_t router, const float* bias,
              int32_t* topk_idx, float* topk_gate, float* scores_opt, void* ws, size_t ws_bytes,
              void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_desc(d));
  MOE_CHECK(need_ptr_t(d, x, "x"));
  MOE_CHECK(need_w(router, d->dense_w_dtype, "router"));
  MOE_CHECK(need_ptr(bias, "bias"));
  MOE_CHECK(need_ptr_t(d, topk_idx, "topk_idx"));
  MOE_CHECK(need_ptr_t(d, topk_gate, "topk_gate"));
  MOE_CHECK(opt_ptr(scores_opt, "scores"));
  MOE_CHECK(check_ws(d, MOE_OP_ROUTE, ws, ws_bytes));
  Plan p;
  LayerWs w{};
  plan_route(d, p, w);
  float* s = scores_opt ? scores_opt : (float*)at(ws, w.s);
  return do_route(d, x, router, bias, topk_idx, topk_gate, s, (float*)at(ws, w.key),
                  (float*)at(ws, w.norms), scores_opt != nullptr, (hipStream_t)stream);
}

int moe_permute(const moe_desc_t* d, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                int32_t* perm_src, int32_t* inv_pos, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_desc(d));
  MOE_CHECK(need_ptr_t(d, topk_idx, "topk_idx"));
  MOE_CHECK(need_ptr(counts, "counts"));
  MOE_CHECK(need_ptr(offsets, "offsets"));
  MOE_CHECK(need_ptr_t(d, perm_src, "perm_src"));
  MOE_CHECK(need_ptr_t(d, inv_pos, "inv_pos"));
  MOE_CHECK(check_ws(d, MOE_OP_PERMUTE, ws, ws_bytes));
  Plan p;
  LayerWs w{};
  plan_permute(d, p, w);
  return do_permute(d, topk_idx, counts, offsets, perm_src, inv_pos, (int32_t*)at(ws, w.blk),
                    (hipStream_t)stream);
}

int moe_latent_down(const moe_desc_t* d, const void* x, moe_w_t lat_down, void* z, void* ws,
                    size_t ws_bytes, void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_desc(d));
  MOE_CHECK(need_ptr_t(d, x, "x"));
  MOE_CHECK(need_w(lat_down, d->latent_w_dtype, "lat_down"));
  MOE_CHECK(need_ptr_t(d, z, "z"));
  MOE_CHECK(check_ws(d, MOE_OP_LATENT_DOWN, ws, ws_bytes));
  Plan p;
  LayerWs lw{};
  plan_latent(d, p, lw);
  return do_latent_down(d, x, lat_down, z, (float*)at(ws, lw.P), at(ws, lw.wld), (hipStream_t)stream);
}

int moe_expert_ffn(const moe_desc_t* d, const void* z, const int32_t* perm_src,
                   const int32_t* offsets, const moe_weights_t* w, void* o_perm, void* ws,
                   size_t ws_bytes, void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_desc(d));
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  MOE_CHECK(need_ptr_t(d, z, "z"));
  MOE_CHECK(need_ptr_t(d, perm_src, "perm_src"));
  MOE_CHECK(need_ptr(offsets, "offsets"));
  MOE_CHECK(need_w(w->exp_gate, d->expert_w_dtype, "exp_gate"));
  MOE_CHECK(need_w(w->exp_up, d->expert_w_dtype, "exp_up"));
  MOE_CHECK(need_w(w->exp_down, d->expert_w_dtype, "exp_down"));
  MOE_CHECK(need_ptr_t(d, o_perm, "o_perm"));
  MOE_CHECK(check_ws(d, MOE_OP_EXPERT_FFN, ws, ws_bytes));
  Plan p;
  LayerWs lw{};
  plan_expert(d, p, lw);
  return do_experts(d, z, perm_src, offsets, w, o_perm, (int32_t*)at(ws, lw.tile_off),
                    (int32_t*)at(ws, lw.tile_info), at(ws, lw.H), mx_bufs(d, ws, lw),
                    (hipStream_t)stream);
}

int moe_expert_gate_up(const moe_desc_t* d, const void* z, const int32_t* perm_src,
                       const int32_t* offsets, const moe_weights_t* w, void* h_out, uint8_t* hq_out,
                       uint8_t* hqs_out, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_desc(d));
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  MOE_CHECK(need_ptr_t(d, z, "z"));
  MOE_CHECK(need_ptr_t(d, perm_src, "perm_src"));
  MOE_CHECK(need_ptr(offsets, "offsets"));
  MOE_CHECK(need_w(w->exp_gate, d->expert_w_dtype, "exp_gate"));
  MOE_CHECK(need_w(w->exp_up, d->expert_w_dtype, "exp_up"));
  const bool q8_out = hq_out != nullptr || hqs_out != nullptr;
  if (q8_out && !d->expert_act_mxfp8)
    return fail(MOE_ERR_INVALID_ARG, "hq_out / hqs_out need expert_act_mxfp8 = 1");
  if (q8_out == (h_out != nullptr) && d->T > 0)
    return fail(MOE_ERR_INVALID_ARG, "give either h_out or both hq_out and hqs_out");
  if (q8_out) {
    MOE_CHECK(need_ptr_t(d, hq_out, "hq_out"));
    if (hqs_out == nullptr && d->T > 0) return fail(MOE_ERR_INVALID_ARG, "hqs_out is NULL");
  } else {
    MOE_CHECK(need_ptr_t(d, h_out, "h_out"));
  }
  MOE_CHECK(check_ws(d, MOE_OP_EXPERT_GATE_UP, ws, ws_bytes));
  Plan p;
  LayerWs lw{};
  plan_gate_up(d, p, lw);
  MxBufs mx;
  if (d->expert_act_mxfp8) {
    mx.zq = (uint8_t*)at(ws, lw.zq);
    mx.zqs = (uint8_t*)at(ws, lw.zqs);
    mx.hq = hq_out;
    mx.hqs = hqs_out;
  }
  return do_gate_up(d, z, perm_src, offsets, w, (int32_t*)at(ws, lw.tile_off),
                    (int32_t*)at(ws, lw.tile_info), h_out, mx, (hipStream_t)stream);
}

int moe_combine(const moe_desc_t* d, const void* o_perm, const int32_t* inv_pos,
                const float* topk_gate, const float* rms_gain, void* n_out, float* u_out_opt,
                void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_desc(d));
  MOE_CHECK(need_ptr_t(d, o_perm, "o_perm"));
  MOE_CHECK(need_ptr_t(d, inv_pos, "inv_pos"));
  MOE_CHECK(need_ptr_t(d, topk_gate, "topk_gate"));
  MOE_CHECK(opt_ptr(rms_gain, "rms_gain"));
  MOE_CHECK(need_ptr_t(d, n_out, "n_out"));
  MOE_CHECK(opt_ptr(u_out_opt, "u_out"));
  return do_combine(d, o_perm, inv_pos, topk_gate, rms_gain, n_out, u_out_opt, (hipStream_t)stream);
}

int moe_output(const moe_desc_t* d, const void* x, const void* n, const moe_weights_t* w, void* y,
               void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_desc(d));
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  MOE_CHECK(need_ptr_t(d, x, "x"));
  MOE_CHECK(need_ptr_t(d, n, "n"));
  MOE_CHECK(need_w(w->lat_up, d->latent_w_dtype, "lat_up"));
  if (d->n_shared > 0) {
    MOE_CHECK(need_w(w->sh_gate, d->dense_w_dtype, "sh_gate"));
    MOE_CHECK(need_w(w->sh_up, d->dense_w_dtype, "sh_up"));
    MOE_CHECK(need_w(w->sh_down, d->dense_w_dtype, "sh_down"));
  }
  MOE_CHECK(need_ptr_t(d, y, "y"));
  MOE_CHECK(check_ws(d, MOE_OP_OUTPUT, ws, ws_bytes));
  Plan p;
  LayerWs lw{};
  plan_output(d, p, lw);
  return do_output(d, x, n, w, y, at(ws, lw.Hs), (float*)at(ws, lw.P), at(ws, lw.wlu),
                   (hipStream_t)stream);
}

int moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, int64_t ld, uint8_t* codes,
                       uint8_t* scales, void* stream) {
  g_last_error.clear();
  if (rows < 0 || K <= 0 || K % 32 || ld < K)
    return fail(MOE_ERR_INVALID_ARG, "rows >= 0, K > 0 with K %% 32 == 0 and ld >= K required");
  if (rows == 0) return MOE_OK;
  if (ld % 8) return fail(MOE_ERR_UNSUPPORTED, "ld must be a multiple of 8 (16-byte rows)");
  MOE_CHECK(need_ptr(x, "x"));
  MOE_CHECK(need_ptr(codes, "codes"));
  if (scales == nullptr) return fail(MOE_ERR_INVALID_ARG, "scales is NULL");
  MOE_LAUNCH(moe::launch_quantize_mx8(x, rows, K, ld, codes, scales, (hipStream_t)stream),
             "quantize_mxfp8");
  return MOE_OK;
}

namespace {
// do the byte ranges [a, a + na) and [b, b + nb) share a byte?
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}
}

int moe_mxfp4_tile(const uint8_t* data, const uint8_t* scale, uint8_t* data_out, uint8_t* scale_out,
                   int64_t rows, int32_t K, void* stream) {
  g_last_error.clear();
  if (rows < 0 || K <= 0 || K % 128 || rows % 64)
    return fail(MOE_ERR_INVALID_ARG, "rows >= 0 with rows %% 64 == 0 and K > 0 with K %% 128 == 0 required");
  if (rows == 0) return MOE_OK;
  MOE_CHECK(need_ptr(data, "data"));
  MOE_CHECK(need_ptr(data_out, "data_out"));
  if (scale == nullptr || scale_out == nullptr) return fail(MOE_ERR_INVALID_ARG, "scale or scale_out is NULL");
  if (((uintptr_t)scale | (uintptr_t)scale_out) % 4)
    return fail(MOE_ERR_INVALID_ARG, "scale and scale_out must be 4-byte aligned");
  const int64_t nd = rows * (K / 2), ns = rows * (K / 32);
  if (overlap(data_out, nd, data, nd) || overlap(data_out, nd, scale, ns) ||
      overlap(scale_out, ns, data, nd) || overlap(scale_out, ns, scale, ns) ||
      overlap(data_out, nd, scale_out, ns))
    return fail(MOE_ERR_INVALID_ARG, "an output overlaps an input or the other output");
  MOE_LAUNCH(moe::launch_tile_mxfp4(data, scale, data_out, scale_out, rows, K, (hipStream_t)stream),
             "mxfp4_tile");
  return MOE_OK;
}

int moe_mxfp4_frag_tiled_bytes(int64_t rows, int32_t K, int64_t* data_bytes, int64_t* scale_bytes) {
  g_last_error.clear();
  if (rows < 0 || K <= 0 || rows % 32 || K % 32)
    return fail(MOE_ERR_INVALID_ARG, "rows >= 0 with rows %% 32 == 0 and K > 0 with K %% 32 == 0 required");
  if (!data_bytes || !scale_bytes) return fail(MOE_ERR_INVALID_ARG, "data_bytes or scale_bytes is NULL");
  moe::tiled_mxfp4_frag_bytes(rows, K, data_bytes, scale_bytes);
  return MOE_OK;
}

int moe_mxfp4_frag_tile(const uint8_t* data, const uint8_t* scale, uint8_t* data_out, uint8_t* scale_out,
                        int64_t rows, int32_t K, void* stream) {
  g_last_error.clear();
  if (rows < 0 || K <= 0 || rows % 32 || K % 32)
    return fail(MOE_ERR_INVALID_ARG, "rows >= 0 with rows %% 32 == 0 and K > 0 with K %% 32 == 0 required");
  if (rows == 0) return MOE_OK;
  MOE_CHECK(need_ptr(data, "data"));
  MOE_CHECK(need_ptr(data_out, "data_out"));
  if (scale == nullptr || scale_out == nullptr) return fail(MOE_ERR_INVALID_ARG, "scale or scale_out is NULL");
  if (((uintptr_t)scale_out) % 4) return fail(MOE_ERR_INVALID_ARG, "scale_out must be 4-byte aligned");
  int64_t nd = 0, ns = 0;
  moe::tiled_mxfp4_frag_bytes(rows, K, &nd, &ns);
  const int64_t id = rows * (K / 2), is = rows * (K / 32);
  if (overlap(data_out, nd, data, id) || overlap(data_out, nd, scale, is) || overlap(scale_out, ns, data, id) ||
      overlap(scale_out, ns, scale, is) || overlap(data_out, nd, scale_out, ns))
    return fail(MOE_ERR_INVALID_ARG, "an output overlaps an input or the other output");
  MOE_LAUNCH(moe::launch_tile_mxfp4_frag(data, scale, data_out, scale_out, rows, K, (hipStream_t)stream),
             "mxfp4_frag_tile");
  return MOE_OK;
}

int64_t moe_bf16_tiled_bytes(int64_t rows, int32_t K) {
  if (rows < 0 || K <= 0 || rows % 32 || K % 8) return 0;
  return moe::tiled_bf16_bytes(rows, K);
}

int moe_bf16_tile(const void* data, void* data_out, int64_t rows, int32_t K, void* stream) {
  g_last_error.clear();
  if (rows < 0 || K <= 0 || rows % 32 || K % 8)
    return fail(MOE_ERR_INVALID_ARG, "rows >= 0 with rows %% 32 == 0 and K > 0 with K %% 8 == 0 required");
  if (rows == 0) return MOE_OK;
  MOE_CHECK(need_ptr(data, "data"));
  MOE_CHECK(need_ptr(data_out, "data_out"));
  if (overlap(data_out, moe::tiled_bf16_bytes(rows, K), data, rows * (int64_t)K * 2))
    return fail(MOE_ERR_INVALID_ARG, "data_out overlaps data");
  MOE_LAUNCH(moe::launch_tile_bf16(data, data_out, rows, K, (hipStream_t)stream), "bf16_tile");
  return MOE_OK;
}

int moe_qb_bias(const moe_desc_t* d, const float* scores, float* bias_out, float* quantile_out,
                void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_desc(d));
  if (d->T == 0) return fail(MOE_ERR_INVALID_ARG, "moe_qb_bias needs T > 0");
  MOE_CHECK(need_ptr(scores, "scores"));
  MOE_CHECK(need_ptr(bias_out, "bias_out"));
  MOE_CHECK(need_ptr(quantile_out, "quantile_out"));
  MOE_LAUNCH(moe::launch_qb_bias(scores, d->T, d->n_experts, d->top_k, quantile_out, bias_out,
                                 (hipStream_t)stream),
             "qb_bias");
  return MOE_OK;
}

int moe_layer_forward(const moe_desc_t* d, const moe_weights_t* w, const void* x, void* y,
                      int32_t* topk_idx_opt, float* topk_gate_opt, int32_t* counts_opt, void* ws,
                      size_t ws_bytes, void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_layer_args(d, w, x, y, topk_idx_opt, topk_gate_opt, counts_opt));
  MOE_CHECK(check_ws(d, MOE_OP_LAYER, ws, ws_bytes));
  SideStream* sd = nullptr;
  MOE_CHECK(side_stream(&sd));
  std::lock_guard<std::mutex> lk(sd->mu);
  return run_layer(d, w, x, y, topk_idx_opt, topk_gate_opt, counts_opt, ws, (hipStream_t)stream, sd,
                   trace_begin());
}

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_layer_forward_noalloc(const moe_desc_t* d, const moe_weights_t* w, const void* x, void* y,
                              int32_t* topk_idx_opt, float* topk_gate_opt, int32_t* counts_opt,
                              void* stream) {
  g_last_error.clear();
  MOE_CHECK(check_layer_args(d, w, x, y, topk_idx_opt, topk_gate_opt, counts_opt));
  const size_t need = ws_bytes_for(d, MOE_OP_LAYER);
  if (need > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_layer_forward_noalloc: this batch needs %zu bytes of scratch, more than the "
                "library's fixed %zu (use moe_layer_forward with a workspace, or fewer tokens)",
                need, kScratchBytes);
  void* ws = nullptr;
  MOE_CHECK(scratch_ptr(&ws));
  return run_layer(d, w, x, y, topk_idx_opt, topk_gate_opt, counts_opt, ws, (hipStream_t)stream,
                   nullptr, Marker{-1});
}

}  // extern "C"
