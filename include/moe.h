/*
 * moe.h -- C ABI of the MI355X (gfx950) Stable LatentMoE layer forward.
 *
 * The layer (pages cited by title and section):
 *   "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか" (lilting.ch)
 *     section "ルーターは計算の割当器":       s = Sigmoid(W_r x); a per-expert
 *       balancing bias is added to s only to choose the top-k; the mixing
 *       weights are the chosen experts' unbiased scores, normalised.
 *     section "K3のエキスパートは896個の小型LLMではない" (its three equations
 *       and flowchart): z = W_down x;  u = sum_{i in TopK} p_i E_i(z);
 *       y = E_1^shared(x) + E_2^shared(x) + W_up RMSNorm(u).
 *   "Kimi K3 テクニカルレポート" (jiwasawa.github.io), section "幅のスケーリング:
 *     Stable LatentMoE": expert activation SiTU-GLU, taken here as
 *     act(g, v) = c*tanh(SiLU(g)/c) * c*tanh(v/c) (c = situ_c).
 *   "Kimi K3 ... Open Frontier Intelligence" (ai-tech-express.jp), section
 *     "MXFP4 Quantization-Aware Training": MXFP4 weights (OCP MX v1.0 e2m1
 *     elements, one e8m0 scale per 32 elements along K).
 *
 * Library state: in device memory only the fixed scratch array of
 * moe_layer_forward_noalloc (one copy per GPU the library runs on). On the
 * host: the per-device side stream of moe_layer_forward (three events with it),
 * the device address of that scratch per GPU, the trace events of
 * moe_trace_enable, and the thread-local error text of moe_last_error.
 *
 * Calling convention (all entry points):
 *   - Every pointer argument is a DEVICE pointer (hipMalloc'd or equivalent)
 *     unless stated; descriptors and weight structs are HOST memory read
 *     during the call only. Device pointers must be 16-byte aligned.
 *   - The caller owns every buffer. The library allocates no device memory:
 *     scratch comes from the caller's workspace `ws` of at least
 *     moe_workspace_bytes(desc, op) bytes (16-byte aligned; NULL allowed when
 *     that size is 0). Calls that share a workspace must be stream-ordered.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Calls only
 *     enqueue work and return; nothing synchronises the host.
 *   - Arguments are validated on the host before any HIP call; a failing call
 *     returns a negative status and enqueues nothing. moe_last_error() gives a
 *     thread-local description. Non-finite input values are not checked; the
 *     results for them are unspecified.
 *
 * Layouts (row-major, K contiguous for every weight, as an [out, in] linear):
 *   x [T, d]            y [T, d]           z, n [T, d_lat]
 *   W_r [E, d]          router_bias [E] fp32
 *   W_ld [d_lat, d]     W_lu [d, d_lat]    rms_gain [d_lat] fp32 (NULL = 1)
 *   W_g, W_v [E, F, d_lat]   W_o [E, d_lat, F]
 *   W_gs, W_vs [S, Fs, d]    W_os [S, d, Fs]
 *   MXFP4 weight [R, K]: data = packed bytes [R, K/2] (element 2i in the low
 *   nibble of byte i, 16-byte aligned like every tensor), scale = e8m0 bytes
 *   [R, K/32] (4-byte aligned).
 *   Tiled MXFP4 weight (routed experts on the MXFP8 path only, see
 *   expert_w_tiled; made by moe_mxfp4_tile; R % 64 == 0, K % 128 == 0): the
 *   same bytes reordered. Packed: byte j (0..63) of row r's 128-element stage
 *   kt (row-major byte 64 kt + j of the row) at ((r/2) (K/128) + kt) 128 +
 *   (r%2) 64 + j, i.e. [R/2][K/128][2][64]: a stage of a row pair is one
 *   128-byte line. Scales: the scale of row r, 32-element block b at
 *   ((r/64) (K/128) + b/4) 256 + (r%64) 4 + b%4, i.e. [R/64][K/128][64][4].
 *   Fragment-tiled bf16 weight (routed experts, see expert_w_tiled; made by
 *   moe_bf16_tile; R % 32 == 0): K padded with zeros to Kp, the next multiple
 *   of 64; for each group g of 32 rows and each k-step s of 16 elements, the
 *   1 KB at byte (g (Kp/16) + s) 1024 holds 64 pieces of 8 elements, piece l
 *   = row 32 g + l % 32, k = 16 s + 8 (l / 32) .. +7 (the order in which the
 *   bf16 matrix instruction takes its B operand). W_g, W_v as R = E F rows of
 *   K = d_latent, W_o as R = E d_latent rows of K = d_ff; moe_bf16_tiled_bytes
 *   gives the size (R Kp 2 bytes).
 *   Fragment-tiled MXFP4 weight (routed experts on the bf16-activation path,
 *   see expert_w_tiled; made by moe_mxfp4_frag_tile; R % 32 == 0, K % 32 ==
 *   0): K padded with zeros to Kp, the next multiple of 128. Packed codes: for
 *   each group g of 32 rows and each 64-element tile t, the 1 KB at byte
 *   (g (Kp/64) + t) 1024 holds 64 pieces of 16 bytes; piece l (row 32 g +
 *   l % 32) holds in its bytes 4s .. 4s+3 the 8 codes of k = 64 t + 16 s +
 *   8 (l / 32) .. +7 (s = 0..3, low nibble first). Scales: for each group g
 *   and 128-element pair p, the 128 bytes at (g (Kp/128) + p) 128 hold, for
 *   each of the 32 rows, the 4 scale bytes of its 32-element blocks 4p .. 4p+3.
 *   moe_mxfp4_frag_tiled_bytes gives both sizes (R Kp/2 and R Kp/32 bytes).
 *   topk_idx [T, k] int32, topk_gate [T, k] fp32 (slot order = key descending,
 *   ties to the lower expert index).
 *   Permutation: rows of expert e are offsets[e] .. offsets[e+1]-1 (offsets has
 *   E+1 entries), ordered by ascending (token, slot); perm_src[row] = t*k + j;
 *   inv_pos[t*k + j] = row.
 *
 * Supported dtype combinations: act = F32 with every weight F32; or act = BF16
 * with router/shared weights BF16 and latent / expert weights BF16 or MXFP4.
 * Other combinations return MOE_ERR_UNSUPPORTED. d, d_lat, F and Fs must be
 * multiples of 32; 1 <= k <= E <= 4096; T >= 0 (T = 0 is an empty batch).
 * Size limits of one call (MOE_ERR_UNSUPPORTED beyond them): T * k <= 2^30,
 * T * k / 128 + E <= 65535, and with bf16 activations z (T * d_lat * 2 bytes)
 * under 2 GiB, since the expert kernels gather its rows with 32-bit offsets;
 * split larger batches into several calls.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* bad dims, NULL or misaligned pointer, k > E, ... */
  MOE_ERR_UNSUPPORTED = -2,   /* valid but not implemented (dtype combination, sizes) */
  MOE_ERR_WORKSPACE = -3,     /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = -4            /* a HIP launch / runtime call failed */
};

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2 } moe_dtype_t;

/* Which entry point a workspace is sized for. */
typedef enum {
  MOE_OP_ROUTE = 0, MOE_OP_PERMUTE = 1, MOE_OP_LATENT_DOWN = 2, MOE_OP_EXPERT_FFN = 3,
  MOE_OP_COMBINE = 4, MOE_OP_OUTPUT = 5, MOE_OP_LAYER = 6, MOE_OP_EXPERT_GATE_UP = 7
} moe_op_t;

typedef struct {
  int32_t T;            /* tokens in the batch */
  int32_t d_model;      /* d */
  int32_t d_latent;     /* d_lat */
  int32_t n_experts;    /* E, routed experts */
  int32_t top_k;        /* k */
  int32_t d_ff;         /* F, routed expert intermediate */
  int32_t n_shared;     /* S, shared experts (may be 0) */
  int32_t d_ff_shared;  /* Fs */
  float situ_c;         /* SiTU-GLU cap c (> 0) */
  float rms_eps;        /* RMSNorm epsilon (>= 0) */
  int32_t act_dtype;      /* x, z, h, o, n, shared h, y: MOE_F32 or MOE_BF16 */
  int32_t expert_w_dtype; /* W_g, W_v, W_o */
  int32_t latent_w_dtype; /* W_ld, W_lu */
  int32_t dense_w_dtype;  /* W_r, W_gs, W_vs, W_os */
  /* 0: the routed experts' GEMMs take z and h in act_dtype (bf16 MFMA on the
     decoded weights). 1: they take z and h quantised to MXFP8 (OCP MX, E4M3
     elements with one e8m0 scale per 32 along K: X = floor(log2 amax) - 8,
     round to nearest even, saturating) and run on gfx950's scaled MFMA
     (MXFP8 x MXFP4); needs act_dtype MOE_BF16, expert_w_dtype MOE_MXFP4 and
     d_latent, d_ff multiples of 128. Changes the numerics (the oracle quantises
     the same way). */
  int32_t expert_act_mxfp8;
  /* 0: W_g, W_v, W_o row-major. 1: tiled, made once per weight set at load
     time (needs act_dtype MOE_BF16):
     - MXFP4 weights with expert_act_mxfp8 = 1: the tiled MXFP4 layout above
       (moe_mxfp4_tile); the scaled-MFMA expert kernels then read each
       128-element K stage as whole 128-byte lines of row pairs and the
       stage's scales of 64 weight rows as 256 contiguous bytes;
     - MXFP4 weights with expert_act_mxfp8 = 0: the fragment-tiled MXFP4
       layout above (moe_mxfp4_frag_tile); the expert kernels load each
       64-element K tile of a weight fragment as one 1 KB line straight into
       registers and decode it there;
     - bf16 weights: the fragment-tiled bf16 layout above (moe_bf16_tile); the
       expert kernels load each weight fragment straight into registers as
       one 1 KB line, without staging it in LDS.
     Same results as the row-major weights in every case. */
  int32_t expert_w_tiled;
} moe_desc_t;

/* A weight tensor: data (dtype of its class) and, for MXFP4 only, scales. */
typedef struct {
  const void* data;
  const uint8_t* scale;
} moe_w_t;

typedef struct {
  moe_w_t router;              /* W_r [E, d] */
  const float* router_bias;    /* b [E] fp32 */
  moe_w_t lat_down;            /* W_ld [d_lat, d] */
  moe_w_t lat_up;              /* W_lu [d, d_lat] */
  const float* rms_gain;       /* [d_lat] fp32, or NULL for a gain of 1 */
  moe_w_t exp_gate, exp_up;    /* W_g, W_v [E, F, d_lat] */
  moe_w_t exp_down;            /* W_o [E, d_lat, F] */
  moe_w_t sh_gate, sh_up;      /* W_gs, W_vs [S, Fs, d] */
  moe_w_t sh_down;             /* W_os [S, d, Fs] */
} moe_weights_t;

/* Bytes of workspace that entry point `op` needs for this descriptor
   (0 for an invalid descriptor; check moe_check_desc first). With MXFP4
   latent maps and a batch whose latent-down / output GEMM runs in one pass
   (at least 256 tiles of 256 x 256), the latent-down, output and layer
   workspaces include a bf16 copy of W_ld / W_up (d_lat x d x 2 bytes each),
   decoded exactly from the MXFP4 weight on every call. */
size_t moe_workspace_bytes(const moe_desc_t* desc, int op);

/* Host-only validation of a descriptor: MOE_OK, MOE_ERR_INVALID_ARG or
   MOE_ERR_UNSUPPORTED. Makes no HIP call. */
int moe_check_desc(const moe_desc_t* desc);

/* Router and top-k ("ルーターは計算の割当器").
   For each token t: l_e = sum_k x[t][k] W_r[e][k] as the fp32 chain
   acc = fma(x, w, acc) over k ascending from +0; s_e = sigmoid(l_e) by the
   library's fixed IEEE-754 fp32 sequence (Cody-Waite reduction + degree-7
   Taylor polynomial + one correctly rounded division); key_e = s_e + b_e.
   topk_idx[t] = the k experts with the largest keys (key descending, ties to
   the lower index); topk_gate[t][j] = s_{idx_j} / (s_{idx_0} + ... + s_{idx_{k-1}})
   in fp32, summed in slot order. scores_opt: if non-NULL receives s [T, E] fp32.
   x: act dtype [T, d]; router.data: dense_w dtype [E, d]. */
int moe_route(const moe_desc_t* desc, const void* x, moe_w_t router, const float* bias,
              int32_t* topk_idx, float* topk_gate, float* scores_opt,
              void* ws, size_t ws_bytes, void* stream);

/* Token permutation: group the T*k (token, slot) pairs by expert (the
   dispatch step of the flowchart: run the chosen experts).
   counts [E], offsets [E+1], perm_src [T*k], inv_pos [T*k] as described in
   the layout notes. Deterministic (no order decided by atomics).
   topk_idx entries outside [0, E) are skipped (they take no row; offsets[E]
   then counts only the valid entries); if a token lists one expert twice,
   both entries get rows, in unspecified order between the two. */
int moe_permute(const moe_desc_t* desc, const int32_t* topk_idx, int32_t* counts,
                int32_t* offsets, int32_t* perm_src, int32_t* inv_pos,
                void* ws, size_t ws_bytes, void* stream);

/* Latent down-projection z = W_down x (equation z = W_down x), stored in the
   act dtype. x [T, d]; z [T, d_lat]; lat_down: latent_w dtype.
   ws: moe_workspace_bytes(desc, MOE_OP_LATENT_DOWN) bytes, which is 0 unless
   the batch is too small to fill the GPU with output tiles; then K is split
   and the fp32 partial sums pass through the workspace (added in a fixed
   order, so results stay deterministic). */
int moe_latent_down(const moe_desc_t* desc, const void* x, moe_w_t lat_down, void* z,
                    void* ws, size_t ws_bytes, void* stream);

/* Routed experts on the permuted rows (E_i(z) of the u equation):
   for every row r of expert e (offsets[e] <= r < offsets[e+1]) with token
   t = perm_src[r] / k: h = act(W_g[e] z_t, W_v[e] z_t) (stored in the act
   dtype), o_perm[r] = W_o[e] h (act dtype, [T*k, d_lat], permuted order).
   Only exp_gate / exp_up / exp_down of `w` are read. perm_src and offsets as
   produced by moe_permute (offsets[E] rows are processed). */
int moe_expert_ffn(const moe_desc_t* desc, const void* z, const int32_t* perm_src,
                   const int32_t* offsets, const moe_weights_t* w, void* o_perm,
                   void* ws, size_t ws_bytes, void* stream);

/* First half of moe_expert_ffn (the gated up-projection of E_i in the u
   equation, with the SiTU-GLU activation of "Kimi K3 テクニカルレポート",
   section "幅のスケーリング: Stable LatentMoE"): for every row r of expert e with
   token t = perm_src[r] / k, h[r] = act(W_g[e] z_t, W_v[e] z_t). Reads exp_gate
   and exp_up of `w`. Output, exactly one of:
     h_out [T*k, F] in the act dtype (permuted rows), or
     hq_out [T*k, F] E4M3 codes and hqs_out [T*k, F/32] e8m0 scale bytes: h
       rounded to bf16 and quantised to MXFP8 by the rule of
       moe_quantize_mxfp8, the form in which moe_expert_ffn passes h to the
       down projection on the scaled-MFMA path (expert_act_mxfp8 = 1 only).
   With expert_act_mxfp8 = 1, z is quantised to MXFP8 first, as in
   moe_expert_ffn. Anything else (both or neither output, hq without hqs, hq
   without expert_act_mxfp8) is MOE_ERR_INVALID_ARG. ws: at least
   moe_workspace_bytes(desc, MOE_OP_EXPERT_GATE_UP) bytes (tile table and the
   MXFP8 copy of z). Rows past offsets[E] are not written. */
int moe_expert_gate_up(const moe_desc_t* desc, const void* z, const int32_t* perm_src,
                       const int32_t* offsets, const moe_weights_t* w, void* h_out,
                       uint8_t* hq_out, uint8_t* hqs_out, void* ws, size_t ws_bytes, void* stream);

/* Weighted combine and RMSNorm (u equation, then RMSNorm of the y equation):
   u_t = sum_j topk_gate[t][j] * o_perm[inv_pos[t*k + j]] (fp32, j ascending);
   n_t = u_t / sqrt(mean(u_t^2) + eps) * gain, stored in the act dtype.
   u_out_opt: if non-NULL receives u [T, d_lat] fp32. */
int moe_combine(const moe_desc_t* desc, const void* o_perm, const int32_t* inv_pos,
                const float* topk_gate, const float* rms_gain, void* n_out, float* u_out_opt,
                void* stream);

/* Output (y equation): y = W_up n + sum_s W_os[s] act(W_gs[s] x, W_vs[s] x),
   accumulated in fp32, stored in the act dtype. Reads lat_up and sh_* of `w`.
   ws holds the shared hidden rows and, for small batches, fp32 split-K
   partials (see moe_latent_down). */
int moe_output(const moe_desc_t* desc, const void* x, const void* n, const moe_weights_t* w,
               void* y, void* ws, size_t ws_bytes, void* stream);

/* The whole layer: route, permute, latent down, experts, combine, output.
   y [T, d] act dtype. Optional outputs (NULL to skip): topk_idx [T, k],
   topk_gate [T, k], counts [E]. The latent down-projection and the shared
   experts' gate/up do not depend on the routing: they run on a second stream
   that the library keeps per device, forked from `stream` with an event at
   the start of the call and joined back into it before the routed experts
   (and, at batches of at most 1024 tokens, where the shared experts' share of
   the output GEMM is also made there, again before the output's final sum),
   so the call remains ordered on `stream` like any other work there.
   Library state behind this call (host side, the only state the library
   keeps besides the thread-local error text and the trace events of
   moe_trace_enable): per device, one non-blocking stream of default priority
   and three events, created by the first call on that device and kept until
   the process ends; a per-device mutex serialises the fork / join of
   concurrent callers. HIP graph capture: after one eager call on the device
   (which creates that stream and its events), the call can be captured on
   `stream` (the fork and the join become graph dependencies); replays give
   the eager result bit for bit (checked on the K3 decode layers, bf16 and
   MXFP8 experts, with eager calls between the replays). */
int moe_layer_forward(const moe_desc_t* desc, const moe_weights_t* w, const void* x, void* y,
                      int32_t* topk_idx_opt, float* topk_gate_opt, int32_t* counts_opt,
                      void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid allocation): the same
   layer as moe_layer_forward, with the same arguments except the workspace.
   Its scratch is a fixed array of moe_noalloc_scratch_bytes() bytes (128 MiB)
   inside the library's code object: one copy on every GPU the library runs
   on, held until the process ends. The call allocates nothing and runs every
   stage in order on `stream` (no second stream, no events, no tracing).
   A batch whose workspace (moe_workspace_bytes(desc, MOE_OP_LAYER)) exceeds
   the array is rejected on the host with MOE_ERR_UNSUPPORTED (at the K3 shape
   that is above about 360 tokens). All calls on one GPU share its array:
   calls that overlap on one GPU (different streams, or host threads) race and
   must be serialised by the caller. Nothing in the array needs clearing
   between calls (every kernel writes what the same call later reads). The
   first call on a device resolves the array's address (hipGetSymbolAddress);
   after it the call can be captured into a HIP graph and replayed, bit for
   bit like the eager call (same check as moe_layer_forward). */
int moe_layer_forward_noalloc(const moe_desc_t* desc, const moe_weights_t* w, const void* x,
                              void* y, int32_t* topk_idx_opt, float* topk_gate_opt,
                              int32_t* counts_opt, void* stream);
size_t moe_noalloc_scratch_bytes(void);

/* MXFP8 quantisation of bf16 rows, the activation format of the scaled-MFMA
   expert path (expert_act_mxfp8; the MX format of "Kimi K3 ... Open Frontier
   Intelligence", section "MXFP4 Quantization-Aware Training", with 8-bit E4M3
   elements): x [rows, K] bf16 with row stride ld elements, K % 32 == 0 ->
   codes [rows, K] E4M3 bytes and scales [rows, K/32] e8m0 bytes, per block of
   32: X = floor(log2 amax) - 8 clamped to [-127, 127] (amax = 0: -127), byte
   X + 127; code = E4M3 nearest to v / 2^X (ties to even), saturating at
   +-448, sign bit when v < 0. Device pointers owned by the caller;
   asynchronous on stream; allocates nothing. */
int moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, int64_t ld, uint8_t* codes,
                       uint8_t* scales, void* stream);

/* Tiled copy of an MXFP4 weight ("Kimi K3 ... Open Frontier Intelligence",
   section "MXFP4 Quantization-Aware Training": e2m1 elements with one e8m0
   scale per 32 along K) for the scaled-MFMA expert path: data [rows, K/2] and
   scale [rows, K/32] row-major in, data_out and scale_out in the tiled order
   given under Layouts. A pure permutation of bytes, made once when a weight
   set is loaded (W_g, W_v as rows = E * F, K = d_latent; W_o as rows =
   E * d_latent, K = d_ff), not per batch. rows % 64 == 0 and K % 128 == 0;
   data pointers 16-byte and scale pointers 4-byte aligned; no output may
   overlap an input or the other output (else MOE_ERR_INVALID_ARG). Device
   memory owned by the caller; asynchronous on stream; allocates nothing.
   rows == 0 does nothing. */
int moe_mxfp4_tile(const uint8_t* data, const uint8_t* scale, uint8_t* data_out, uint8_t* scale_out,
                   int64_t rows, int32_t K, void* stream);

/* Fragment-tiled copy of an MXFP4 expert weight (layout under Layouts) for
   the expert kernels that decode the weights in registers (bf16 activations,
   expert_act_mxfp8 = 0; "Kimi K3 ... Open Frontier Intelligence", section
   "MXFP4 Quantization-Aware Training"): data [rows, K/2] and scale [rows, K/32]
   row-major in; data_out and scale_out of the sizes moe_mxfp4_frag_tiled_bytes
   gives. A reordering of the same codes and scales (K padded with code 0 and
   scale byte 0), made once when a weight set is loaded. rows % 32 == 0,
   K % 32 == 0; data pointers 16-byte and scale_out 4-byte aligned; no output
   may overlap an input or the other output (else MOE_ERR_INVALID_ARG). Device
   memory owned by the caller; asynchronous on stream; allocates nothing. */
int moe_mxfp4_frag_tile(const uint8_t* data, const uint8_t* scale, uint8_t* data_out, uint8_t* scale_out,
                        int64_t rows, int32_t K, void* stream);
/* Sizes of that copy (host only): *data_bytes = rows Kp / 2, *scale_bytes =
   rows Kp / 32 with Kp = K rounded up to a multiple of 128. */
int moe_mxfp4_frag_tiled_bytes(int64_t rows, int32_t K, int64_t* data_bytes, int64_t* scale_bytes);

/* Fragment-tiled copy of a bf16 expert weight (layout under Layouts) for the
   bf16 expert kernels that keep the weights in registers: data [rows, K]
   row-major in, data_out of moe_bf16_tiled_bytes(rows, K) bytes out (K padded
   with zeros to a multiple of 64). A reordering of the same values, made once
   when a weight set is loaded, not per batch. rows % 32 == 0, K % 8 == 0,
   both pointers 16-byte aligned, data_out not overlapping data (else
   MOE_ERR_INVALID_ARG). Device memory owned by the caller; asynchronous on
   stream; allocates nothing. rows == 0 does nothing. */
int moe_bf16_tile(const void* data, void* data_out, int64_t rows, int32_t K, void* stream);
/* Bytes of that copy: rows * Kp * 2 (0 for invalid rows / K). Host only. */
int64_t moe_bf16_tiled_bytes(int64_t rows, int32_t K);

/* Quantile Balancing: the per-expert selection bias from quantiles of the
   router scores ("Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか",
   section "ルーター専用の独立訓練はない": the boundary at which each expert
   receives its target number of tokens is a quantile of its score
   distribution, and the selection bias is updated from it; "Kimi K3
   テクニカルレポート", section "幅のスケーリング: Stable LatentMoE": quantiles
   taken directly from score histograms). For a batch of T = desc->T tokens
   and target c = round(T k / E) (ties up, clamped to [1, T]):
     quantile_out[e] = the c-th largest scores[t][e] over t   (exact),
     tau             = fp32(sum_e quantile_out[e] / E)         (fp64 sum, e ascending),
     bias_out[e]     = fp32(tau - quantile_out[e]).
   scores [T, E] fp32 (the unbiased sigmoid scores, e.g. moe_route's scores
   output), bias_out [E] and quantile_out [E] fp32: device pointers owned by
   the caller. T must be > 0 (MOE_ERR_INVALID_ARG otherwise). Non-finite
   scores are not supported. Asynchronous on stream; allocates nothing. */
int moe_qb_bias(const moe_desc_t* desc, const float* scores, float* bias_out, float* quantile_out,
                void* stream);

/* Stage tracing. moe_trace_enable(max_calls) makes the next max_calls calls of
   moe_layer_forward record a HIP event before and after each stage, on the
   stream the stage runs on (max_calls = 0 turns tracing off). moe_trace_read
   waits for those events, writes the average milliseconds of each stage over
   the traced calls into ms[0 .. min(max_stages, MOE_TRACE_STAGES)) and the
   number of traced calls into *ncalls, then starts a new trace window. Stage i
   is named by moe_trace_stage_name(i). Stages on the second stream (latent
   down, shared gate/up) overlap the routing stages, so the stage times can add
   up to more than the call. The events are created by the library on the
   device current at moe_trace_enable and live until the next enable.
   moe_trace_enable_stages(max_calls, stage_mask) records only the stages whose
   bit (1 << i) is set in stage_mask (each recorded event can cost a few
   microseconds of the call); moe_trace_read then reports -1 for the others.
   moe_trace_enable(n) is moe_trace_enable_stages(n, all stages). A mask with
   bits past the last stage is MOE_ERR_INVALID_ARG. */
#define MOE_TRACE_STAGES 10
int moe_trace_enable(int max_calls);
int moe_trace_enable_stages(int max_calls, unsigned stage_mask);
int moe_trace_read(float* ms, int max_stages, int* ncalls);
const char* moe_trace_stage_name(int stage);

/* Static text of a status code. */
const char* moe_status_string(int status);

/* Thread-local text of the last failure in this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
