"""GPU parity on seeded random layer shapes: 24 small layers whose sizes,
expert counts, top-k, shared-expert counts, bias laws and weight formats are
drawn from a fixed seed (bf16, MXFP4 weights, and MXFP4 weights with MXFP8
expert inputs in turn, each with row-major and tiled expert weights
alternately). Every token is checked: routing bit-exact, gates
within 1e-6 relative, y within the tolerance of its format."""
import numpy as np
import pytest

import oracle
import synth
from synth.configs import LayerConfig

from _gpu_helpers import say, to64, run_layer, check_y, check_gates

pytestmark = pytest.mark.gpu

KINDS = ("bf16", "mxfp4", "mx8")


def draw(i: int) -> LayerConfig:
    r = np.random.default_rng(1000 + i)
    kind = KINDS[i % 3]

    def mult(lo, hi, step):
        return int(r.integers(lo // step, hi // step + 1)) * step

    d = mult(64, 512, 32)
    d_lat = mult(128, 384, 128) if kind == "mx8" else mult(32, 384, 32)
    F = mult(128, 512, 128) if kind == "mx8" else mult(32, 512, 32)
    E = int(r.integers(1, 201))
    k = int(r.integers(1, min(E, 16) + 1))
    T = int(r.integers(1, 301))
    S = int(r.integers(0, 3))
    Fs = mult(32, 256, 32)
    bias = ("zipf", 1.1, 0.5) if r.random() < 0.25 else ("uniform", float(r.choice([0.0, 0.05, 0.2])))
    kw = {} if kind == "bf16" else dict(expert_w="mxfp4", latent_w="mxfp4")
    if kind == "mx8":
        kw["expert_act"] = "mxfp8"
    if (i // 3) % 2:
        kw["expert_layout"] = "tiled"
    return LayerConfig(f"rnd{i}_{kind}", T=T, d=d, d_lat=d_lat, E=E, k=k, F=F, S=S, Fs=Fs,
                       seed=500 + i, bias=bias, **kw)


CASES = [draw(i) for i in range(24)]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_random_layer(cfg, device):
    say(f"{cfg.name}: T={cfg.T} d={cfg.d} d_lat={cfg.d_lat} E={cfg.E} k={cfg.k} F={cfg.F} "
        f"S={cfg.S} Fs={cfg.Fs} bias={cfg.bias}")
    inp = synth.device_inputs(cfg, device)
    y, idx, gate, counts = run_layer(cfg, inp, device)
    y_ref, inter = oracle.forward(cfg, synth.HostWeights(cfg), keep=True)
    assert np.array_equal(idx.cpu().numpy(), inter["idx"]), "expert indices differ"
    check_gates(gate.cpu().numpy(), inter["p"])
    assert np.array_equal(counts.cpu().numpy(), np.bincount(inter["idx"].ravel(), minlength=cfg.E))
    check_y(cfg, to64(y), y_ref)
