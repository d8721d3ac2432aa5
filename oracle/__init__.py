"""CPU oracle of the Stable LatentMoE layer forward.

TEST INFRASTRUCTURE ONLY: the plain, slow, obviously correct definition of
what the layer computes, used by the test suite, the smoke check and the
benchmark's CPU-baseline leg. The product (the HIP library and its binding)
never imports it, and it imports nothing from the product. Inputs come from
the shared seeded generator (``synth``), or from explicit arrays.

What it computes, step by step (pages cited by title and section):

  "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか" (lilting.ch)
    - section "ルーターは計算の割当器": s = Sigmoid(W_r x) over the E experts;
      a per-expert balancing bias is added to the scores for choosing the
      top-k only; the mixing weights p are the chosen experts' original
      scores, normalised.                                    -> route()
    - section "K3のエキスパートは896個の小型LLMではない", its three equations:
      z = W_down x;  u = sum_{i in TopK} p_i E_i(z);
      y = E_1^shared(x) + E_2^shared(x) + W_up RMSNorm(u);  and its flowchart
      (scores -> top 16 -> run those FFNs -> weighted combine). -> forward()
  "Kimi K3 テクニカルレポート" (jiwasawa.github.io), section "幅のスケーリング:
      Stable LatentMoE": the GLU activation is SiTU-GLU, a soft-capped SwiGLU;
      its closed form c*tanh(SiLU(g)/c) * c*tanh(v/c), c = 8, is fixed by the
      workload specification.                                -> oracle.c
  "Kimi K3 ... Open Frontier Intelligence" (ai-tech-express.jp), section
      "MXFP4 Quantization-Aware Training": MXFP4 weights, decoded exactly.

Readings where the pages are silent:
  * bias is added to the sigmoid score s (not the logit); key = fp32(s + b).
  * ties among keys go to the lower expert index; idx[t] lists the chosen
    experts by key descending (same rule).
  * "normalised" = divided by their sum: S = s_idx0 + s_idx1 + ... (fp32, slot
    order), p_j = s_idx_j / S (fp32).
  * router arithmetic is fixed: fp32 fmaf chain over k ascending from +0, then
    the IEEE-only sigmoid of oracle.c (the choice is discrete, so both sides
    must take it in the same precision).
  * experts are gated FFNs: h = act(W_g z, W_v z), o = W_o h; shared experts
    use the same activation and are summed ungated.
  * RMSNorm: u / sqrt(mean(u^2) + eps) * gain, mean over d_lat.
  * storage points z, h, o, n and the shared activations are rounded to the
    activation dtype; y is kept unrounded (fp64).
  * permutation: rows grouped by expert (ascending expert), inside a group by
    ascending (token, slot); perm_src[row] = t*k + j, inv_pos[t*k + j] = row.
"""
from __future__ import annotations

import ctypes
import os
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")

STORE_F32, STORE_BF16 = 0, 1


@lru_cache(maxsize=None)
def lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    vp, i64, i32, f32, f64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                              ctypes.c_double)
    L.orc_init_constants.argtypes = []
    L.orc_init_constants.restype = None
    L.orc_init_constants()
    sigs = {
        "orc_widen_bf16": ([vp, i64, vp], None),
        "orc_dequant_mxfp4": ([vp, vp, i64, i64, vp], None),
        "orc_sigmoid": ([f32], f32),
        "orc_router": ([vp, vp, vp, i64, i64, i64, vp, vp], None),
        "orc_round_bf16": ([f64], f64),
        "orc_store": ([f64, i32], f64),
        "orc_store_array": ([vp, i64, i32], None),
        "orc_linear": ([vp, i64, i64, vp, i64, vp], None),
        "orc_situ_glu": ([f64, f64, f64], f64),
        "orc_glu": ([vp, vp, i64, f64, i32, vp], None),
        "orc_rmsnorm": ([vp, i64, i64, f64, vp, i32, vp], None),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# --------------------------------------------------------------------------
# storage decoding (exact)
# --------------------------------------------------------------------------

def widen(raw) -> np.ndarray:
    """('f32'|'bf16'|'mxfp4', data) -> float32 array with the exact stored values."""
    kind, data = raw
    if kind == "f32":
        return _c(data, np.float32)
    if kind == "bf16":
        u = _c(data, np.uint16)
        out = np.empty(u.shape, dtype=np.float32)
        lib().orc_widen_bf16(_p(u), u.size, _p(out))
        return out
    if kind == "mxfp4":
        packed, scales = (_c(a, np.uint8) for a in data)
        rows, half = packed.shape[0], packed.shape[-1]
        rows = packed.size // half
        out = np.empty((rows, half * 2), dtype=np.float32)
        lib().orc_dequant_mxfp4(_p(packed), _p(scales), rows, half * 2, _p(out))
        return out.reshape(*packed.shape[:-1], half * 2)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def sigmoid(l) -> np.ndarray:
    """Canonical fp32 sigmoid, elementwise (scalar loop; for tests)."""
    l = np.asarray(l, dtype=np.float32)
    f = lib().orc_sigmoid
    return np.array([f(float(v)) for v in l.ravel()], dtype=np.float32).reshape(l.shape)


def router(x: np.ndarray, Wr: np.ndarray, b: np.ndarray):
    """s, key [T, E] fp32 (logits by the fixed fp32 chain, then sigmoid, + bias)."""
    x = _c(x, np.float32)
    Wr = _c(Wr, np.float32)
    b = _c(b, np.float32)
    T, d = x.shape
    E = Wr.shape[0]
    s = np.empty((T, E), dtype=np.float32)
    key = np.empty((T, E), dtype=np.float32)
    if T:
        lib().orc_router(_p(x), _p(Wr), _p(b), T, d, E, _p(s), _p(key))
    return s, key


def topk(key: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, by key descending, ties to the lower
    index: a stable sort of -key keeps equal keys in index order."""
    order = np.argsort(-key, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gates(s: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """p_j = s_idx_j / (s_idx_0 + s_idx_1 + ...), all fp32, sum in slot order."""
    sel = np.take_along_axis(s, idx.astype(np.int64), axis=1).astype(np.float32)
    tot = np.zeros(sel.shape[0], dtype=np.float32)
    for j in range(sel.shape[1]):
        tot = (tot + sel[:, j]).astype(np.float32)
    return (sel / tot[:, None]).astype(np.float32)


def route(x, Wr, b, k):
    s, key = router(x, Wr, b)
    idx = topk(key, k)
    p = gates(s, idx)
    return {"s": s, "key": key, "idx": idx, "p": p}


def permute(idx: np.ndarray, E: int):
    """Counting sort of the (token, slot) pairs by expert.
    counts[e]; offsets = exclusive scan (E+1 entries); perm_src[row] = t*k + j
    with rows of expert e at offsets[e]..offsets[e+1]-1 in ascending (t, j);
    inv_pos[t*k + j] = row."""
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    nxt = offsets[:-1].copy()
    perm_src = np.empty(T * k, dtype=np.int64)
    inv_pos = np.empty(T * k, dtype=np.int64)
    for a in range(T * k):          # a = t*k + j visited in ascending (t, j)
        e = flat[a]
        perm_src[nxt[e]] = a
        inv_pos[a] = nxt[e]
        nxt[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32), perm_src.astype(np.int32),
            inv_pos.astype(np.int32))


# --------------------------------------------------------------------------
# fp64 forward
# --------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# MXFP8 (OCP MX, E4M3 elements) activations for the scaled-MFMA expert path
# ("Kimi K3 ... Open Frontier Intelligence", section "MXFP4 Quantization-Aware
# Training": 4-bit MX weights; the matrix cores that take MX weights also take
# the activations in an MX format, here 8-bit E4M3 with one power-of-two scale
# per 32 elements along K)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of an OCP FP8 E4M3 code (bias 7; exponent field 0 = subnormal;
    0x7F / 0xFF are NaN)."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def _exp2_floor(a: np.ndarray) -> np.ndarray:
    """floor(log2 |a|) of nonzero finite values (numpy frexp: a = f 2^e, 0.5 <= |f| < 1)."""
    return np.frexp(a)[1].astype(np.int64) - 1


def mx8_quantize(a: np.ndarray):
    """Rows of K values (K % 32 == 0) -> (E4M3 codes uint8 [rows, K], e8m0 scale
    bytes uint8 [rows, K/32]). Per 32-element block: X = floor(log2 amax) - 8
    (8 = the largest E4M3 exponent), clamped to [-127, 127], amax = 0 gives
    X = -127; byte = X + 127. Element: y = v / 2^X (exact), rounded to nearest
    even on the E4M3 grid, saturating at +-448; sign bit set when v < 0."""
    a = np.asarray(a, dtype=np.float64)
    rows, K = a.shape
    blk = a.reshape(rows, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    X = np.full(amax.shape, -127, np.int64)
    nz = amax > 0
    X[nz] = np.clip(_exp2_floor(amax[nz]) - 8, -127, 127)
    y = np.abs(blk) * np.ldexp(1.0, -X)[..., None]
    code = np.zeros(y.shape, np.int64)
    sub = y < 2.0 ** -6
    # subnormal range: multiples of 2^-9 (q = 8 is the first normal, code 0x08)
    code[sub] = np.rint(y[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    e = _exp2_floor(np.where(nrm, y, 1.0))
    m = np.rint((y * np.ldexp(1.0, -e) - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code_n = ((e + 7) << 3) | m
    code_n = np.where((y >= E4M3_MAX) | (code_n > 0x7E), 0x7E, code_n)
    code[nrm] = code_n[nrm]
    code = code | np.where(blk < 0, 0x80, 0)
    return code.reshape(rows, K).astype(np.uint8), (X + 127).astype(np.uint8)


def mx8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E4M3 codes [rows, K] with e8m0 bytes [rows, K/32] -> float64 values."""
    table = np.array([e4m3_value(c) for c in range(256)], np.float64)
    rows, K = codes.shape
    v = table[codes.astype(np.int64)].reshape(rows, K // 32, 32)
    v = v * np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    return v.reshape(rows, K)


def qb_target(T: int, E: int, k: int) -> int:
    """Target tokens per expert: round(T k / E) (ties up), clamped to [1, T]."""
    c = (T * k + E // 2) // E
    return max(1, min(T, c))


def qb_bias(scores: np.ndarray, k: int):
    """Quantile Balancing ("Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何が
    ズレるか", section "ルーター専用の独立訓練はない"; "Kimi K3 テクニカルレポート",
    section "幅のスケーリング: Stable LatentMoE"): each expert's boundary is the
    quantile of its score distribution at which it receives its target number
    of tokens, and the selection bias is set from it.

    scores [T, E] float32 -> (q [E], b [E]) float32: q[e] = the c-th largest
    scores[:, e] (c = qb_target), tau = fp32(sequential fp64 sum of q over e
    ascending / E), b[e] = fp32(tau - q[e])."""
    T, E = scores.shape
    c = qb_target(T, E, k)
    q = np.empty(E, np.float32)
    for e in range(E):
        q[e] = np.sort(scores[:, e])[::-1][c - 1]
    total = 0.0
    for e in range(E):
        total += float(q[e])
    tau = np.float32(total / E)
    b = (tau - q).astype(np.float32)
    return q, b


def linear(A: np.ndarray, W: np.ndarray) -> np.ndarray:
    """A [n, K] (fp64) times W^T, W [N, K] fp32 -> [n, N] fp64 (plain sums)."""
    A = _c(A, np.float64)
    W = _c(W, np.float32)
    n, K = A.shape
    N = W.shape[0]
    out = np.empty((n, N), dtype=np.float64)
    if n and N:
        lib().orc_linear(_p(A), n, K, _p(W), N, _p(out))
    return out


def store(v: np.ndarray, storage: int) -> np.ndarray:
    v = _c(v, np.float64).copy()
    lib().orc_store_array(_p(v), v.size, storage)
    return v


def glu(G: np.ndarray, V: np.ndarray, c: float, storage: int) -> np.ndarray:
    G = _c(G, np.float64)
    V = _c(V, np.float64)
    H = np.empty_like(G)
    lib().orc_glu(_p(G), _p(V), G.size, c, storage, _p(H))
    return H


def situ_glu(g, v, c):
    f = lib().orc_situ_glu
    return f(float(g), float(v), float(c))


def rmsnorm(u: np.ndarray, eps: float, gain, storage: int) -> np.ndarray:
    u = _c(u, np.float64)
    rows, D = u.shape
    out = np.empty_like(u)
    g = None if gain is None else _c(gain, np.float32)
    lib().orc_rmsnorm(_p(u), rows, D, eps, _p(g), storage, _p(out))
    return out


class ArrayWeights:
    """Explicit weights for small hand-built layers: a dict of float32 arrays
    under the names x, W_r, W_ld, W_lu, W_g, W_v, W_o, W_gs, W_vs, W_os, b, gain."""

    def __init__(self, arrays: dict):
        self.a = {k: np.asarray(v) for k, v in arrays.items() if v is not None}

    def raw(self, name, row0=0, rows=None):
        arr = self.a[name]
        arr2 = arr.reshape(-1, arr.shape[-1])
        if rows is None:
            rows = arr2.shape[0] - row0
        return "f32", arr2[row0:row0 + rows]

    def bias(self):
        return self.a["b"].astype(np.float32)

    def gain(self):
        return self.a.get("gain")


def _storage(act: str) -> int:
    return STORE_BF16 if act == "bf16" else STORE_F32


def route_layer(cfg, w, tokens=None):
    """Routing of the layer: full token set, or the listed tokens only (a
    token's routing depends on that token alone)."""
    X = _x_rows(cfg, w, tokens)
    Wr = widen(w.raw("W_r"))
    return route(X, Wr, w.bias(), cfg.k)


def _x_rows(cfg, w, tokens):
    if tokens is None:
        return widen(w.raw("x"))
    tokens = np.asarray(tokens, dtype=np.int64)
    return np.concatenate([widen(w.raw("x", int(t), 1)) for t in tokens], axis=0) \
        if len(tokens) else np.zeros((0, cfg.d), dtype=np.float32)


def forward(cfg, w, tokens=None, routing=None, keep=False):
    """y (fp64, unrounded) for the listed tokens (all if None).

    cfg: dims (d, d_lat, E, k, F, S, Fs), c, eps, act dtype.
    w:   weight source with .raw(name, row0, rows), .bias(), .gain().
    routing: optional dict with 'idx' and 'p' rows for these tokens (else routed here).
    keep: also return intermediates: z (stored), z_in [n, d_lat] and h [n, k, F]
          (the routed experts' gate/up input and down input of every (token,
          slot), after the MXFP8 quantisation when the expert inputs are
          MXFP8), o [n, k, d_lat], u, n (stored), hs [n, S, Fs] (the shared
          experts' stored activations) and the routing."""
    storage = _storage(cfg.act)
    X = _x_rows(cfg, w, tokens).astype(np.float64)
    n_tok = X.shape[0]
    if routing is None:
        routing = route(X.astype(np.float32), widen(w.raw("W_r")), w.bias(), cfg.k)
    idx, p = routing["idx"], routing["p"]

    # z = W_down x, stored
    z = store(linear(X, widen(w.raw("W_ld"))), storage)

    # routed experts, expert by expert: o[t, j] = W_o[e] act(W_g[e] z_t, W_v[e] z_t);
    # with MXFP8 expert inputs, z rows and h rows are quantised first (the same
    # codes the scaled-MFMA path multiplies)
    mx_act = getattr(cfg, "expert_act", "act") == "mxfp8"
    o = np.zeros((n_tok, cfg.k, cfg.d_lat), dtype=np.float64)
    if keep:
        z_in = np.zeros((n_tok, cfg.d_lat), dtype=np.float64)
        h_all = np.zeros((n_tok, cfg.k, cfg.F), dtype=np.float64)
    for e in np.unique(idx):
        rows_t, rows_j = np.nonzero(idx == e)
        e = int(e)
        Wg = widen(w.raw("W_g", e * cfg.F, cfg.F))
        Wv = widen(w.raw("W_v", e * cfg.F, cfg.F))
        Wo = widen(w.raw("W_o", e * cfg.d_lat, cfg.d_lat))
        Z = z[rows_t]
        if mx_act:
            Z = mx8_dequantize(*mx8_quantize(Z))
        H = glu(linear(Z, Wg), linear(Z, Wv), cfg.c, storage)
        if mx_act:
            H = mx8_dequantize(*mx8_quantize(H))
        o[rows_t, rows_j] = store(linear(H, Wo), storage)
        if keep:
            z_in[rows_t] = Z
            h_all[rows_t, rows_j] = H

    # u = sum_j p_j o_j (slot order), n = RMSNorm(u)
    u = np.zeros((n_tok, cfg.d_lat), dtype=np.float64)
    for j in range(cfg.k):
        u = u + p[:, j].astype(np.float64)[:, None] * o[:, j]
    n = rmsnorm(u, cfg.eps, w.gain(), storage)

    # y = W_up n + sum_s shared_s(x)
    y = linear(n, widen(w.raw("W_lu")))
    hs_all = np.zeros((n_tok, cfg.S, cfg.Fs), dtype=np.float64) if keep else None
    for s_ in range(cfg.S):
        Wgs = widen(w.raw("W_gs", s_ * cfg.Fs, cfg.Fs))
        Wvs = widen(w.raw("W_vs", s_ * cfg.Fs, cfg.Fs))
        Wos = widen(w.raw("W_os", s_ * cfg.d, cfg.d))
        Hs = glu(linear(X, Wgs), linear(X, Wvs), cfg.c, storage)
        y = y + linear(Hs, Wos)
        if keep:
            hs_all[:, s_] = Hs
    if keep:
        return y, {"z": z, "z_in": z_in, "h": h_all, "u": u, "n": n, "o": o, "hs": hs_all,
                   "idx": idx, "p": p}
    return y
