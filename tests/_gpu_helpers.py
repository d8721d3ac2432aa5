"""Shared pieces of the GPU parity tests (not collected by pytest).

Tolerances (the bar the GPU path is held to):
  routing (expert indices, counts, permutation order): bit-exact
  gates: within 1e-6 relative (the fixed fp32 sequence makes them bit-exact here)
  y: max |y_gpu - y_oracle| <= TOL * RMS(y_oracle), TOL = 2e-2 for bf16,
     5e-2 for MXFP4 weights, 1e-4 for the all-fp32 layer.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
import sparse_mixture_experts_sigmoid_amd as moe

TOL_BF16, TOL_MX, TOL_F32 = 2e-2, 5e-2, 1e-4
GATE_REL = 1e-6


def tol_of(cfg):
    if cfg.act == "f32":
        return TOL_F32
    if cfg.expert_w == "mxfp4" or cfg.latent_w == "mxfp4":
        return TOL_MX
    return TOL_BF16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def act_torch(cfg):
    return torch.float32 if cfg.act == "f32" else torch.bfloat16


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_layer(cfg, inp, dev="cuda:0"):
    desc = moe.make_desc(cfg)
    y = torch.empty((cfg.T, cfg.d), dtype=act_torch(cfg), device=dev)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    counts = torch.empty((cfg.E,), dtype=torch.int32, device=dev)
    ws = moe.workspace(desc, moe.MOE_OP_LAYER, dev)
    moe.moe_layer_forward(desc, moe.prepare_weights(cfg, inp), inp["x"], y, idx, gate, counts, ws)
    torch.cuda.synchronize()
    return y, idx, gate, counts


def check_gates(g_gpu: np.ndarray, g_ref: np.ndarray):
    rel = np.abs(g_gpu.astype(np.float64) - g_ref.astype(np.float64)) / np.abs(g_ref).clip(1e-30)
    assert rel.max() <= GATE_REL, f"gate rel err {rel.max():.3e}"


def check_y(cfg, y_gpu: np.ndarray, y_ref: np.ndarray, what=""):
    rms = float(np.sqrt((y_ref ** 2).mean()))
    err = float(np.abs(y_gpu - y_ref).max())
    tol = tol_of(cfg)
    say(f"  {cfg.name}{what}: max|dy| = {err / rms:.3e} x RMS (tol {tol:g}), RMS {rms:.4f}")
    assert err <= tol * rms, f"{cfg.name}{what}: max|dy|/RMS = {err / rms:.3e} > {tol}"


def sample_tokens(cfg, idx: np.ndarray, n: int, seed: int = 0) -> np.ndarray:
    """A seeded token sample that includes tokens routed to the hottest and the
    coldest non-empty expert, plus the first and last token."""
    rng = np.random.default_rng(seed)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    hot = int(np.argmax(counts))
    nz = np.nonzero(counts)[0]
    cold = int(nz[np.argmin(counts[nz])])
    picks = {0, cfg.T - 1}
    for e in (hot, cold):
        picks.add(int(np.nonzero((idx == e).any(1))[0][0]))
    rest = rng.choice(cfg.T, size=min(n, cfg.T), replace=False)
    for t in rest:
        if len(picks) >= n:
            break
        picks.add(int(t))
    return np.array(sorted(picks), dtype=np.int64)


def staged_front(cfg, inp, dev="cuda:0"):
    """Routing, permutation and z of a layer through the staged entry points:
    (desc, idx, gate, offsets, perm_src, inv_pos, z)."""
    desc = moe.make_desc(cfg)
    T, k, E = cfg.T, cfg.k, cfg.E
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    moe.moe_route(desc, inp["x"], inp["W_r"], inp["b"], idx, gate, None,
                  moe.workspace(desc, moe.MOE_OP_ROUTE, dev))
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    moe.moe_permute(desc, idx, counts, offsets, perm, inv, moe.workspace(desc, moe.MOE_OP_PERMUTE, dev))
    z = torch.empty((T, cfg.d_lat), dtype=act_torch(cfg), device=dev)
    moe.moe_latent_down(desc, inp["x"], inp["W_ld"], z, moe.workspace(desc, moe.MOE_OP_LATENT_DOWN, dev))
    return desc, idx, gate, offsets, perm, inv, z


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (normal range; 2^-133 below it)."""
    e = np.frexp(np.abs(np.asarray(v, np.float64)))[1]
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def check_mx8_layer(cfg, y_gpu, y_ref, z_gpu, z_ref, what=""):
    """End-to-end check of a layer whose experts take MXFP8 z (rows = tokens).

    The MXFP8 code of a z element is an integer decided by floating point: a
    z computed with fp32 accumulation (GPU) and one with fp64 (oracle) may
    differ by one bf16 step, and where that step crosses an E4M3 rounding
    midpoint the two codes differ by one E4M3 step. Both codes are correct
    quantisations of an admissible z. So: every z element must be within one
    bf16 step (plus 2^-12 RMS(z) near zero) of the oracle's; tokens whose z quantises identically on both
    sides must meet the tolerance; tokens with a code flip are counted (at most
    2 % of them) and only guarded against gross error (0.25 x RMS); their
    values on the oracle's own z are checked exactly by check on the staged path
    (experts, combine, output on the oracle's z)."""
    # one bf16 step of the value, plus 2^-12 of RMS(z) for elements near zero
    # (where the fp32-vs-fp64 difference of a 7168-term sum spans many steps
    # of a tiny value)
    dz = np.abs(z_gpu - z_ref)
    zr = float(np.sqrt((z_ref ** 2).mean()))
    bound = bf16_ulp(z_ref) + 2.0 ** -12 * zr
    assert (dz <= bound).all(), (f"{cfg.name}{what}: z differs by {float((dz / bound).max()):.2f} x "
                                 f"(one bf16 step + 2^-12 RMS(z))")
    cg, sg = oracle.mx8_quantize(z_gpu)
    co, so = oracle.mx8_quantize(z_ref)
    flip = ((cg != co).any(1)) | ((sg != so).any(1))
    rms = float(np.sqrt((y_ref ** 2).mean()))
    err = np.abs(y_gpu - y_ref).max(1) / rms
    tol = tol_of(cfg)
    agree_max = float(err[~flip].max()) if (~flip).any() else 0.0
    flip_max = float(err[flip].max()) if flip.any() else 0.0
    say(f"  {cfg.name}{what}: {int(flip.sum())} of {len(err)} tokens with an MXFP8 z code flip "
        f"(max|dy| {flip_max:.3e} x RMS); the others max|dy| = {agree_max:.3e} x RMS (tol {tol:g})")
    assert agree_max <= tol, f"{cfg.name}{what}: max|dy|/RMS = {agree_max:.3e} > {tol}"
    assert flip.mean() <= 0.02, f"{cfg.name}{what}: {int(flip.sum())} tokens with z code flips"
    assert flip_max <= 0.25, f"{cfg.name}{what}: a flipped token is off by {flip_max:.3e} x RMS"


def staged_on_z(cfg, inp, x, z, dev="cuda:0"):
    """y of the tokens x [n, d] through the staged entry points, with the
    latent z [n, d_lat] given (instead of computed by moe_latent_down)."""
    c = cfg.replace(T=x.shape[0])
    desc = moe.make_desc(c)
    T, k, E = c.T, c.k, c.E
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    moe.moe_route(desc, x, inp["W_r"], inp["b"], idx, gate, None, moe.workspace(desc, moe.MOE_OP_ROUTE, dev))
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    moe.moe_permute(desc, idx, counts, offsets, perm, inv, moe.workspace(desc, moe.MOE_OP_PERMUTE, dev))
    o = torch.empty((T * k, c.d_lat), dtype=act_torch(c), device=dev)
    moe.moe_expert_ffn(desc, z, perm, offsets, inp, o, moe.workspace(desc, moe.MOE_OP_EXPERT_FFN, dev))
    n = torch.empty((T, c.d_lat), dtype=act_torch(c), device=dev)
    moe.moe_combine(desc, o, inv, gate, inp["gain"], n)
    y = torch.empty((T, c.d), dtype=act_torch(c), device=dev)
    moe.moe_output(desc, x, n, inp, y, moe.workspace(desc, moe.MOE_OP_OUTPUT, dev))
    torch.cuda.synchronize()
    return y, idx
