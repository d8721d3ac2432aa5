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
