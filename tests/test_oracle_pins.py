"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own code: each checks it against a
brute force, a closed form, an invariant, or a special case that reduces to a
textbook formula (routing, gates, permutation, SiTU-GLU limits, RMSNorm,
MXFP4 decoding, the dense-mixture and single-FFN reductions of the layer)."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from synth.configs import LayerConfig

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_ulp_diff(a, b):
    """Distance in fp32 ulps between two same-sign finite fp32 arrays."""
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


# --------------------------------------------------------------------------
# router pieces
# --------------------------------------------------------------------------

def test_sigmoid_within_2ulp_of_fp64():
    rng = np.random.default_rng(0)
    l = np.concatenate([np.linspace(-20, 20, 40001), rng.uniform(-20, 20, 20000),
                        rng.normal(0, 1, 20000)]).astype(np.float32)
    s = oracle.sigmoid(l)
    ref = (1.0 / (1.0 + np.exp(-l.astype(np.float64)))).astype(np.float32)
    assert f32_ulp_diff(s, ref).max() <= 2


def test_sigmoid_special_values_and_monotone():
    assert oracle.sigmoid([0.0])[0] == np.float32(0.5)
    assert oracle.sigmoid([-0.0])[0] == np.float32(0.5)
    l = np.sort(np.random.default_rng(1).uniform(-30, 30, 50000).astype(np.float32))
    s = oracle.sigmoid(l)
    assert np.all(np.diff(s) >= 0)
    assert oracle.sigmoid([30.0])[0] == np.float32(1.0)
    assert 0 < oracle.sigmoid([-30.0])[0] < 1e-12


def _bf16_valued(rng, shape, scale):
    v = (rng.normal(0, scale, shape)).astype(np.float32)
    u = v.view(np.uint32) & np.uint32(0xFFFF0000)     # truncate to a bf16 value
    return u.view(np.float32)


def test_router_logit_chain_order_and_bias():
    """With bf16-valued operands every product is exact in fp32, so the fixed
    chain acc = fmaf(x_k, w_k, acc) (k ascending from +0) equals a plain fp32
    running sum; s must be the canonical sigmoid of it and key = fp32(s + b)."""
    rng = np.random.default_rng(2)
    T, d, E = 5, 300, 7
    x = _bf16_valued(rng, (T, d), 1.0)
    W = _bf16_valued(rng, (E, d), 1 / math.sqrt(d))
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    s, key = oracle.router(x, W, b)
    acc = np.zeros((T, E), dtype=np.float32)
    for kk in range(d):
        acc = (acc + (x[:, kk:kk + 1] * W[:, kk][None, :]).astype(np.float32)).astype(np.float32)
    assert np.array_equal(s, oracle.sigmoid(acc))
    assert np.array_equal(key, (s + b[None, :]).astype(np.float32))
    # a reversed summation order gives different bits somewhere (the order is pinned)
    acc_r = np.zeros((T, E), dtype=np.float32)
    for kk in reversed(range(d)):
        acc_r = (acc_r + (x[:, kk:kk + 1] * W[:, kk][None, :]).astype(np.float32)).astype(np.float32)
    assert not np.array_equal(acc, acc_r)


def _brute_topk(keys, k):
    """Largest ordered k-tuple under (key desc, index asc), by exhaustion."""
    E = len(keys)
    best = None
    for tup in itertools.permutations(range(E), k):
        rank = tuple((float(keys[i]), -i) for i in tup)
        if best is None or rank > best[0]:
            best = (rank, tup)
    return list(best[1])


def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(3)
    n = 0
    for E in range(1, 8):
        for k in range(1, E + 1):
            for _ in range(6):
                keys = (rng.integers(0, 4, size=(1, E)) * 0.25).astype(np.float32)  # many ties
                got = oracle.topk(keys, k)[0].tolist()
                assert got == _brute_topk(keys[0], k), (E, k, keys)
                n += 1
    assert n > 100


def test_gates_sum_and_independence_from_bias():
    cfg = synth.config(0)
    w = synth.HostWeights(cfg)
    r = oracle.route_layer(cfg, w)
    p = r["p"].astype(np.float64)
    assert np.all(p >= 0)
    assert np.abs(p.sum(1) - 1).max() <= cfg.k * 2.0 ** -24
    # gates use the unbiased scores: recomputing them from s alone gives the same bits
    assert np.array_equal(oracle.gates(r["s"], r["idx"]), r["p"])
    # pushing every unselected expert's bias down keeps idx (and its order) and p
    b = w.bias().copy()
    sel = np.zeros((cfg.T, cfg.E), bool)
    np.put_along_axis(sel, r["idx"].astype(np.int64), True, axis=1)
    never = ~sel.any(0)
    if never.any():
        b2 = b.copy()
        b2[never] -= 0.5
        r2 = oracle.route(oracle.widen(w.raw("x")), oracle.widen(w.raw("W_r")), b2, cfg.k)
        assert np.array_equal(r2["idx"], r["idx"]) and np.array_equal(r2["p"], r["p"])
    # and bias does move the selection: a huge bias on expert 0 puts it first everywhere
    b3 = b.copy()
    b3[0] = 10.0
    r3 = oracle.route(oracle.widen(w.raw("x")), oracle.widen(w.raw("W_r")), b3, cfg.k)
    assert np.all(r3["idx"][:, 0] == 0)
    assert np.array_equal(oracle.gates(r["s"], r3["idx"]), r3["p"])


def test_gate_single_expert_is_one():
    s = np.array([[0.3, 0.9, 0.2]], np.float32)
    idx = np.array([[1]], np.int32)
    assert oracle.gates(s, idx)[0, 0] == np.float32(1.0)


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (37, 9, 3), (64, 32, 4), (200, 50, 7)])
def test_permutation_properties(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.permute(idx, E)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.all(np.diff(offsets) == counts)
    assert np.array_equal(np.sort(perm), np.arange(T * k))
    assert np.array_equal(inv[perm], np.arange(T * k))
    for e in range(E):
        grp = perm[offsets[e]:offsets[e + 1]]
        assert np.all(idx.reshape(-1)[grp] == e)
        assert np.all(np.diff(grp // k) > 0)          # strictly ascending tokens
    # same order as a library lexicographic sort on (expert, t*k + j)
    a = np.arange(T * k)
    assert np.array_equal(perm, np.lexsort((a, idx.reshape(-1))))
    # permute then un-permute is the identity on rows broadcast over k
    x = rng.normal(size=(T, 5))
    xp = x[perm // k]
    back = xp[inv].reshape(T, k, 5)
    assert np.array_equal(back, np.repeat(x[:, None, :], k, axis=1))


# --------------------------------------------------------------------------
# SiTU-GLU, RMSNorm, bf16 rounding
# --------------------------------------------------------------------------

def test_situ_glu_limits_and_symmetry():
    rng = np.random.default_rng(4)
    for g, v in rng.normal(0, 3, size=(200, 2)):
        silu = g / (1 + math.exp(-g))
        # c -> infinity: SwiGLU SiLU(g) * v, error O((x/c)^2) relative
        big = oracle.situ_glu(g, v, 1e6)
        assert abs(big - silu * v) <= 1e-9 * (1 + abs(silu * v))
        # zero up-branch gives zero; odd in v
        assert oracle.situ_glu(g, 0.0, 8.0) == 0.0
        assert oracle.situ_glu(g, -v, 8.0) == -oracle.situ_glu(g, v, 8.0)
        # soft cap on both branches (|act| < c^2; fp64 tanh reaches 1.0 exactly far out)
        assert abs(oracle.situ_glu(g * 100, v * 100, 8.0)) <= 64.0
        assert abs(oracle.situ_glu(g, v, 8.0)) < 64.0
    assert oracle.situ_glu(0.0, 5.0, 8.0) == 0.0          # SiLU(0) = 0
    # deep saturation: both tanh factors -> 1, product -> c^2 = 64
    assert abs(oracle.situ_glu(1e3, 1e3, 8.0) - 64.0) < 1e-9
    assert abs(oracle.situ_glu(1e3, -1e3, 8.0) + 64.0) < 1e-9
    # large negative gate: SiLU -> 0-, product -> 0
    assert abs(oracle.situ_glu(-60.0, 1.0, 8.0)) < 1e-20


def test_rmsnorm_invariants():
    rng = np.random.default_rng(5)
    u = rng.normal(0, 3, size=(6, 128))
    n = oracle.rmsnorm(u, 1e-6, None, oracle.STORE_F32)
    rms = np.sqrt((n ** 2).mean(1))
    assert np.allclose(rms, 1.0, atol=1e-6)
    n2 = oracle.rmsnorm(7.5 * u, 1e-6, None, oracle.STORE_F32)
    assert np.allclose(n, n2, rtol=1e-6, atol=1e-7)
    assert np.all(oracle.rmsnorm(np.zeros((1, 16)), 1e-6, None, 0) == 0)
    g = rng.uniform(0.5, 2, 128).astype(np.float32)
    ng = oracle.rmsnorm(u, 1e-6, g, oracle.STORE_F32)
    assert np.allclose(ng, (n * g[None, :]), rtol=1e-6)


def _bf16_round_exact(v: float) -> float:
    """Brute force: nearest value with 8 significant bits, ties to even significand."""
    if v == 0:
        return 0.0
    fv = Fraction(v)
    e = math.floor(math.log2(abs(v)))
    while Fraction(2) ** e > abs(fv):
        e -= 1
    while Fraction(2) ** (e + 1) <= abs(fv):
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    lo = math.floor(fv / q)
    cand = [lo, lo + 1]
    best = min(cand, key=lambda m: (abs(fv - m * q), m % 2))
    return float(best * q)


def test_bf16_rounding_brute_force():
    rng = np.random.default_rng(6)
    vals = list(rng.normal(0, 10, 3000)) + list(rng.normal(0, 1e-3, 500))
    # exact ties: 1 + 2^-8 (between 1 and 1+2^-7) goes to even (1.0); 1 + 3*2^-8 goes up
    vals += [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2.0 ** -130 * 1.5, 3.0]
    for v in vals:
        assert oracle.lib().orc_round_bf16(float(v)) == _bf16_round_exact(float(v)), v
    assert oracle.lib().orc_round_bf16(1 + 2 ** -8) == 1.0
    assert oracle.lib().orc_round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6


# --------------------------------------------------------------------------
# MXFP4 decoding and the generator's quantiser
# --------------------------------------------------------------------------

def test_mxfp4_decode_matches_spec_table():
    spec = json.load(open(os.path.join(GOLDEN, "ocp_e2m1.json")))
    vals = spec["e2m1_code_to_value"]
    for scale_byte in (127, 120, 130, 1, 200):
        for code in range(16):
            packed = np.full((1, 16), code | (code << 4), np.uint8)
            scales = np.full((1, 1), scale_byte, np.uint8)
            out = oracle.widen(("mxfp4", (packed, scales)))
            want = vals[code] * 2.0 ** (scale_byte - spec["e8m0_bias"])
            assert np.all(out == np.float32(want)), (code, scale_byte)
    # element 2i sits in the low nibble of byte i
    packed = np.zeros((1, 16), np.uint8)
    packed[0, 0] = 0x72                                  # elem0 = code 2 (1.0), elem1 = code 7 (6.0)
    out = oracle.widen(("mxfp4", (packed, np.full((1, 1), 127, np.uint8))))
    assert out[0, 0] == 1.0 and out[0, 1] == 6.0 and np.all(out[0, 2:] == 0)


def test_mxfp4_quantiser_error_bound():
    """Generator's quantiser vs the oracle's decoder: every element is within
    half a grid step of its bf16 master, or saturated at 6 * 2^X."""
    cfg = synth.config(4)
    K = 256
    sig = synth.sigma_of(cfg, "W_g")
    packed, scales = synth.host_mxfp4(cfg.seed, 6, 0, 64, K, sig)
    deq = oracle.widen(("mxfp4", (packed, scales))).astype(np.float64)
    master = oracle.widen(("bf16", synth.host_normal(cfg.seed, 6, 0, 64 * K, sig, "bf16")))
    master = master.reshape(64, K).astype(np.float64)
    X = scales.astype(np.int64).repeat(32, axis=1) - 127
    q = np.abs(master) / 2.0 ** X
    step = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0)) * 2.0 ** X
    err = np.abs(deq - master)
    sat = q > 6
    assert np.all(err[~sat] <= step[~sat] / 2 + 0)
    assert np.all(np.abs(deq[sat]) == 6 * 2.0 ** X[sat])
    # the block maximum sits in [4, 8) * 2^X, so it is not crushed to zero
    amax = np.abs(master).reshape(64, K // 32, 32).max(-1)
    assert np.all(amax / 2.0 ** (scales.astype(np.int64) - 127) >= 4)
    # grid values (times the block scale) survive a quantise -> decode round trip
    assert np.array_equal(deq[~sat & (err == 0)], master[~sat & (err == 0)])


def test_generator_slices_are_counter_based():
    a = synth.host_normal(7, 3, 0, 1000, 0.5, "bf16")
    b = synth.host_normal(7, 3, 123, 500, 0.5, "bf16")
    assert np.array_equal(a[123:623], b)
    f = synth.host_normal(7, 3, 0, 200000, 1.0, "f32").astype(np.float64)
    assert abs(f.mean()) < 0.01 and abs(f.std() - 1) < 0.01
    assert not np.array_equal(synth.host_normal(8, 3, 0, 100, 1.0, "f32"),
                              synth.host_normal(7, 3, 0, 100, 1.0, "f32"))


# --------------------------------------------------------------------------
# the layer: reductions to textbook forms
# --------------------------------------------------------------------------

def _small_cfg(**kw):
    base = dict(name="t", T=16, d=32, d_lat=32, E=4, k=4, F=24, S=0, Fs=16, seed=0,
                act="f32", expert_w="f32", latent_w="f32", dense_w="f32", bias=("zero",))
    base.update(kw)
    return LayerConfig(**base)


def _act(g, v, c):
    silu = g / (1 + np.exp(-g))
    return c * np.tanh(silu / c) * c * np.tanh(v / c)


def _rand_arrays(cfg, rng, identity_latents=False):
    f = lambda *s: rng.normal(0, 1 / math.sqrt(s[-1]), s).astype(np.float32)
    a = {
        "x": rng.normal(0, 1, (cfg.T, cfg.d)).astype(np.float32),
        "W_r": f(cfg.E, cfg.d),
        "W_ld": np.eye(cfg.d_lat, cfg.d, dtype=np.float32) if identity_latents else f(cfg.d_lat, cfg.d),
        "W_lu": np.eye(cfg.d, cfg.d_lat, dtype=np.float32) if identity_latents else f(cfg.d, cfg.d_lat),
        "W_g": f(cfg.E, cfg.F, cfg.d_lat), "W_v": f(cfg.E, cfg.F, cfg.d_lat),
        "W_o": f(cfg.E, cfg.d_lat, cfg.F),
        "W_gs": f(max(cfg.S, 1), cfg.Fs, cfg.d), "W_vs": f(max(cfg.S, 1), cfg.Fs, cfg.d),
        "W_os": f(max(cfg.S, 1), cfg.d, cfg.Fs),
        "b": rng.uniform(-0.1, 0.1, cfg.E).astype(np.float32), "gain": None,
    }
    return a


def test_dense_mixture_reduction():
    """k = E, identity latent maps, no shared experts: the layer is
    RMSNorm(sum_e (s_e / sum s) FFN_e(x)), a dense mixture."""
    cfg = _small_cfg()
    rng = np.random.default_rng(7)
    a = _rand_arrays(cfg, rng, identity_latents=True)
    y = oracle.forward(cfg, oracle.ArrayWeights(a))
    x = a["x"].astype(np.float64)
    s = 1 / (1 + np.exp(-(x @ a["W_r"].astype(np.float64).T)))
    mix = np.zeros_like(x)
    for e in range(cfg.E):
        ffn = _act(x @ a["W_g"][e].T.astype(np.float64), x @ a["W_v"][e].T.astype(np.float64),
                   cfg.c) @ a["W_o"][e].T.astype(np.float64)
        mix += (s[:, e] / s.sum(1))[:, None] * ffn
    ref = mix / np.sqrt((mix ** 2).mean(1, keepdims=True) + cfg.eps)
    assert np.abs(y - ref).max() <= 2e-5 * np.sqrt((ref ** 2).mean())


def test_single_expert_is_one_ffn():
    """E = k = 1, identity latents, no shared experts: y = RMSNorm(FFN(x))."""
    cfg = _small_cfg(E=1, k=1, F=40)
    rng = np.random.default_rng(8)
    a = _rand_arrays(cfg, rng, identity_latents=True)
    y, inter = oracle.forward(cfg, oracle.ArrayWeights(a), keep=True)
    assert np.all(inter["p"] == 1.0)
    x = a["x"].astype(np.float64)
    ffn = _act(x @ a["W_g"][0].T.astype(np.float64), x @ a["W_v"][0].T.astype(np.float64),
               cfg.c) @ a["W_o"][0].T.astype(np.float64)
    ref = ffn / np.sqrt((ffn ** 2).mean(1, keepdims=True) + cfg.eps)
    assert np.abs(y - ref).max() <= 2e-5 * np.sqrt((ref ** 2).mean())


def test_output_is_sum_of_shared_and_routed_parts():
    cfg = _small_cfg(d=48, d_lat=32, E=6, k=2, S=2, Fs=20)
    rng = np.random.default_rng(9)
    a = _rand_arrays(cfg, rng)
    y = oracle.forward(cfg, oracle.ArrayWeights(a))
    a_noup = dict(a, W_lu=np.zeros_like(a["W_lu"]))
    y_shared = oracle.forward(cfg, oracle.ArrayWeights(a_noup))
    y_routed = oracle.forward(cfg.replace(S=0), oracle.ArrayWeights(a))
    assert np.allclose(y, y_shared + y_routed, rtol=1e-12, atol=1e-12)
    # shared part by hand: sum_s W_os act(W_gs x, W_vs x)
    x = a["x"].astype(np.float64)
    ref = sum(_act(x @ a["W_gs"][s].T.astype(np.float64), x @ a["W_vs"][s].T.astype(np.float64),
                   cfg.c) @ a["W_os"][s].T.astype(np.float64) for s in range(cfg.S))
    assert np.abs(y_shared - ref).max() <= 1e-5 * np.abs(ref).max()


def test_token_permutation_equivariance():
    cfg = synth.config(0)
    w = synth.HostWeights(cfg)
    full = {n: oracle.widen(w.raw(n)) for n in ("x", "W_r", "W_ld", "W_lu", "W_g", "W_v", "W_o",
                                              "W_gs", "W_vs", "W_os")}
    for n, shp in (("W_g", (cfg.E, cfg.F, cfg.d_lat)), ("W_v", (cfg.E, cfg.F, cfg.d_lat)),
                   ("W_o", (cfg.E, cfg.d_lat, cfg.F)), ("W_gs", (cfg.S, cfg.Fs, cfg.d)),
                   ("W_vs", (cfg.S, cfg.Fs, cfg.d)), ("W_os", (cfg.S, cfg.d, cfg.Fs))):
        full[n] = full[n].reshape(shp)
    full["b"] = w.bias()
    full["gain"] = w.gain()
    y, inter = oracle.forward(cfg, oracle.ArrayWeights(full), keep=True)
    y_gen = oracle.forward(cfg, w)
    assert np.array_equal(y, y_gen)                      # same inputs either way
    perm = np.random.default_rng(10).permutation(cfg.T)
    fp = dict(full, x=full["x"][perm])
    y2, inter2 = oracle.forward(cfg, oracle.ArrayWeights(fp), keep=True)
    assert np.array_equal(inter2["idx"], inter["idx"][perm])
    assert np.allclose(y2, y[perm], rtol=0, atol=0)


def test_token_subset_equals_full_rows():
    cfg = synth.config(0)
    w = synth.HostWeights(cfg)
    y = oracle.forward(cfg, w)
    sub = [0, 5, 63, 17]
    ys = oracle.forward(cfg, w, tokens=sub)
    assert np.array_equal(ys, y[sub])


def test_k3_table_shapes():
    """The 3-matrix expert reading reproduces the pages' parameter total."""
    t = json.load(open(os.path.join(GOLDEN, "k3_table.json")))
    cfg = synth.config("k3_prefill")
    assert (cfg.d, cfg.E, cfg.k, cfg.S, cfg.d_lat, cfg.F) == (
        t["d_model"], t["routed_experts_per_layer"], t["experts_per_token"],
        t["shared_experts"], t["latent_dim"], t["expert_intermediate"])
    per_layer = (cfg.E * 3 * cfg.d_lat * cfg.F + cfg.S * 3 * cfg.d * cfg.Fs
                 + 2 * cfg.d * cfg.d_lat + cfg.E * cfg.d)
    total = t["layers"] * per_layer
    assert abs(total - t["total_params"]) / t["total_params"] < 0.005
    # a 2-matrix (ungated) expert would miss the total by about a third
    per_layer2 = (cfg.E * 2 * cfg.d_lat * cfg.F + cfg.S * 2 * cfg.d * cfg.Fs
                  + 2 * cfg.d * cfg.d_lat + cfg.E * cfg.d)
    assert abs(t["layers"] * per_layer2 - t["total_params"]) / t["total_params"] > 0.3


# ---------------------------------------------------------------------------
# Quantile Balancing bias
# ---------------------------------------------------------------------------

def test_qb_target_hand_values():
    # 16384 tokens x top-16 over 896 experts: 292.57 tokens per expert -> 293
    assert oracle.qb_target(16384, 896, 16) == 293
    assert oracle.qb_target(64, 32, 4) == 8          # exactly 8
    assert oracle.qb_target(1, 4, 2) == 1            # 0.5 rounds up
    assert oracle.qb_target(3, 1, 1) == 3            # one expert takes every token
    assert oracle.qb_target(2, 64, 1) == 1           # never below one token


@pytest.mark.parametrize("T,E,k,grid", [(50, 7, 3, None), (40, 5, 2, 8), (9, 3, 1, 2), (1, 4, 4, None)])
def test_qb_quantile_is_the_order_statistic(T, E, k, grid):
    """q[e] is the c-th largest score: fewer than c scores lie strictly above
    it and at least c lie at or above it (checked by counting, with heavy ties
    when the scores sit on a coarse grid)."""
    rng = np.random.default_rng(T * 100 + E)
    s = rng.random((T, E)).astype(np.float32)
    if grid:
        s = (np.floor(s * grid) / grid + 1.0 / (2 * grid)).astype(np.float32)
    q, b = oracle.qb_bias(s, k)
    c = oracle.qb_target(T, E, k)
    for e in range(E):
        above = int((s[:, e] > q[e]).sum())
        at_or_above = int((s[:, e] >= q[e]).sum())
        assert above < c <= at_or_above, (e, above, c, at_or_above)
        assert q[e] in s[:, e]


def test_qb_bias_centred_and_shifts_quantiles_to_one_boundary():
    rng = np.random.default_rng(7)
    s = (1.0 / (1.0 + np.exp(-rng.standard_normal((300, 40))))).astype(np.float32)
    q, b = oracle.qb_bias(s, 4)
    tau = np.float32(sum(float(v) for v in q) / 40)
    # every expert's boundary lands on the common value tau (up to one rounding)
    assert np.all(np.abs((q + b).astype(np.float64) - float(tau)) <= np.spacing(np.float32(1.0)))
    assert abs(float(b.astype(np.float64).mean())) < 1e-6
    # experts with higher quantiles get lower bias, in the same order
    assert np.array_equal(np.argsort(q, kind="stable"), np.argsort(-b, kind="stable"))


def test_qb_hand_example():
    # 4 tokens, 2 experts, k = 1: target round(4/2) = 2 tokens per expert
    s = np.array([[0.9, 0.1], [0.8, 0.2], [0.7, 0.6], [0.3, 0.4]], np.float32)
    q, b = oracle.qb_bias(s, 1)
    assert q.tolist() == [np.float32(0.8), np.float32(0.4)]
    tau = np.float32((float(np.float32(0.8)) + float(np.float32(0.4))) / 2)
    assert b.tolist() == [np.float32(tau - np.float32(0.8)), np.float32(tau - np.float32(0.4))]
    # with the bias, each expert's top-2 scores are the ones at or above its boundary
    key = s + b
    assert ((key >= tau).sum(axis=0) == 2).all()


# ---------------------------------------------------------------------------
# MXFP8 (E4M3) activation quantiser of the scaled-MFMA expert path
# ---------------------------------------------------------------------------

def test_e4m3_value_table():
    # OCP E4M3: bias 7, 3 mantissa bits, subnormal step 2^-9, max 448 (0x7E)
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x44) == 3.0
    assert oracle.e4m3_value(0xC0) == -2.0
    assert np.isnan(oracle.e4m3_value(0x7F))
    vals = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))      # codes 0..0x7E increase


def test_mx8_grid_values_round_trip():
    """Every finite E4M3 value, placed in a block whose amax fixes the scale
    2^X, comes back exactly."""
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)] +
                    [oracle.e4m3_value(c) for c in range(0x80, 0xFF)])
    for X in (-3, 0, 5):
        v = np.zeros((1, 32 * 8))
        v[0, :len(grid)] = grid * 2.0 ** X
        v[0, 31] = 448.0 * 2.0 ** X          # amax of block 0 -> X
        for b in range(1, 8):
            v[0, 32 * b + 31] = 448.0 * 2.0 ** X
        codes, scales = oracle.mx8_quantize(v)
        assert (scales == X + 127).all()
        assert np.array_equal(oracle.mx8_dequantize(codes, scales), v)


def test_mx8_scale_rule_and_bounds():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((40, 128)) * np.exp(rng.uniform(-6, 6, (40, 1)))
    codes, scales = oracle.mx8_quantize(v)
    blk = np.abs(v).reshape(40, 4, 32).max(axis=2)
    # X = floor(log2 amax) - 8, by the textbook route (math.frexp per block)
    import math
    want = np.array([[math.frexp(a)[1] - 1 - 8 + 127 for a in row] for row in blk])
    assert np.array_equal(scales.astype(int), want)
    d = oracle.mx8_dequantize(codes, scales)
    X = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    # half a step: 2^-4 relative in the normal range, 2^(X-10) absolute below it;
    # above 448 * 2^X (amax lies in [256, 512) * 2^X) the element saturates
    err = np.abs(d - v)
    cap = 448.0 * 2.0 ** X
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** (X - 10))
    bound = np.where(np.abs(v) > cap, np.abs(v) - cap, bound)
    assert (err <= bound * (1 + 1e-12)).all()
    assert (np.abs(d) <= cap).all()
    assert ((v < 0) == (codes >= 0x80)).all()


def test_mx8_ties_saturation_and_zero():
    one = np.zeros((1, 32))
    one[0, 0] = 256.0                        # amax 2^8 -> X = 0
    one[0, 1] = 1.0 + 1.0 / 16               # midway 1 and 1.125 -> even (1.0)
    one[0, 2] = 1.0 + 3.0 / 16               # midway 1.125 and 1.25 -> even (1.25)
    one[0, 3] = 2.0 ** -10                   # midway 0 and 2^-9 -> even (0)
    one[0, 4] = 3 * 2.0 ** -10               # midway 2^-9 and 2^-8 -> even (2^-8)
    one[0, 5] = -(2.0 ** -12)                # tiny negative -> -0
    codes, scales = oracle.mx8_quantize(one)
    assert scales[0, 0] == 127
    assert codes[0, 1] == 0x38 and codes[0, 2] == 0x3A
    assert codes[0, 3] == 0x00 and codes[0, 4] == 0x02 and codes[0, 5] == 0x80
    sat = np.zeros((1, 32))
    sat[0, 0] = 511.0                        # amax in [256, 512): X = 0, 511 > 448
    codes, scales = oracle.mx8_quantize(sat)
    assert scales[0, 0] == 127 and codes[0, 0] == 0x7E
    codes, scales = oracle.mx8_quantize(np.zeros((2, 64)))
    assert (codes == 0).all() and (scales == 0).all()


# --------------------------------------------------------------------------
# storage points: which intermediates the oracle rounds, and to what
# --------------------------------------------------------------------------

def _bf16_representable(v):
    """Exactly a bf16 value: an fp32 value whose low 16 mantissa bits are zero."""
    v = np.asarray(v, np.float64)
    f = v.astype(np.float32)
    return (f.astype(np.float64) == v) & ((f.view(np.uint32) & 0xFFFF) == 0)


def _f32_representable(v):
    v = np.asarray(v, np.float64)
    return v.astype(np.float32).astype(np.float64) == v


def _bf16_half_ulp(v):
    """Half the spacing of bf16 values at |v| (normal range)."""
    e = np.frexp(np.abs(np.asarray(v, np.float64)))[1]     # |v| in [2^(e-1), 2^e)
    return np.ldexp(1.0, e - 1 - 8)


def _routed_rows(inter, cfg):
    """(token, slot) pairs in use (every slot of every token)."""
    return inter["o"].reshape(-1, cfg.d_lat), inter["h"].reshape(-1, cfg.F)


PIN_BF16 = LayerConfig("pin_bf16", T=24, d=64, d_lat=64, E=6, k=2, F=32, S=2, Fs=32, seed=5,
                       bias=("uniform", 0.05))
PIN_MX8 = LayerConfig("pin_mx8", T=24, d=64, d_lat=128, E=5, k=2, F=128, S=1, Fs=32, seed=6,
                      expert_w="mxfp4", latent_w="mxfp4", expert_act="mxfp8", bias=("uniform", 0.05))


def test_storage_points_bf16():
    """bf16 activations: z, h, o, n and the shared experts' h are stored in bf16
    (each one exactly a bf16 value, none of them all zero), z and n by rounding
    to nearest (within half a bf16 step of the unrounded fp64 value, computed
    here with numpy's matmul); y is not rounded."""
    cfg = PIN_BF16
    w = synth.HostWeights(cfg)
    y, inter = oracle.forward(cfg, w, keep=True)
    o, h = _routed_rows(inter, cfg)
    for name, v in (("z", inter["z"]), ("h", h), ("o", o), ("n", inter["n"]), ("hs", inter["hs"])):
        assert np.abs(v).max() > 0, name
        assert _bf16_representable(v).all(), f"{name} is not stored in bf16"
    assert np.array_equal(inter["z_in"], inter["z"]), "bf16 experts take z as stored"
    x = oracle.widen(w.raw("x")).astype(np.float64)
    z_exact = x @ oracle.widen(w.raw("W_ld")).astype(np.float64).T
    assert (np.abs(inter["z"] - z_exact) <= _bf16_half_ulp(z_exact) * (1 + 1e-9)).all()
    u = inter["u"]
    n_exact = u / np.sqrt((u ** 2).mean(1, keepdims=True) + cfg.eps)
    assert (np.abs(inter["n"] - n_exact) <= _bf16_half_ulp(n_exact) * (1 + 1e-9)).all()
    assert not _bf16_representable(y).all(), "y is returned unrounded"


def test_storage_points_fp32():
    """fp32 activations: the same intermediates are fp32 values, and most of
    them are not on the bf16 grid (nothing is rounded to bf16)."""
    cfg = synth.config("tiny_f32")
    y, inter = oracle.forward(cfg, synth.HostWeights(cfg), keep=True)
    o, h = _routed_rows(inter, cfg)
    for name, v in (("z", inter["z"]), ("h", h), ("o", o), ("n", inter["n"]), ("hs", inter["hs"])):
        assert _f32_representable(v).all(), f"{name} is not stored in fp32"
        nz = v[v != 0]
        assert (~_bf16_representable(nz)).mean() > 0.9, f"{name} looks rounded to bf16"


def test_storage_points_mxfp8_expert_inputs():
    """MXFP8 expert inputs: the z rows and h rows the experts multiply are MXFP8
    values (quantising them again changes nothing), they differ from the bf16
    values they came from (the quantisation took place), and o, n and the
    shared h stay bf16."""
    cfg = PIN_MX8
    y, inter = oracle.forward(cfg, synth.HostWeights(cfg), keep=True)
    o, h = _routed_rows(inter, cfg)
    for name, v in (("z_in", inter["z_in"]), ("h", h)):
        assert np.abs(v).max() > 0, name
        again = oracle.mx8_dequantize(*oracle.mx8_quantize(v))
        assert np.array_equal(again, v), f"{name} is not an MXFP8 value"
    assert _bf16_representable(inter["z"]).all()
    assert not np.array_equal(inter["z_in"], inter["z"]), "z was not quantised"
    # bf16 h of the same rows, recomputed from the quantised z (numpy matmul);
    # the kept h must be its MXFP8 image, not the bf16 value itself
    w = synth.HostWeights(cfg)
    idx = inter["idx"]
    t, j = 3, 1
    e = int(idx[t, j])
    Wg = oracle.widen(w.raw("W_g", e * cfg.F, cfg.F)).astype(np.float64)
    Wv = oracle.widen(w.raw("W_v", e * cfg.F, cfg.F)).astype(np.float64)
    zt = inter["z_in"][t]
    g, v = Wg @ zt, Wv @ zt
    hb = np.array([oracle.lib().orc_round_bf16(c * math.tanh(gg / (1 + math.exp(-gg)) / c) *
                                               c * math.tanh(vv / c))
                   for gg, vv, c in zip(g, v, [cfg.c] * len(g))])
    hq = oracle.mx8_dequantize(*oracle.mx8_quantize(hb[None, :]))[0]
    assert np.array_equal(inter["h"][t, j], hq)
    assert not np.array_equal(hq, hb)
    for name, v in (("o", o), ("n", inter["n"]), ("hs", inter["hs"])):
        assert _bf16_representable(v).all(), f"{name} is not stored in bf16"
