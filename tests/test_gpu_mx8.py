"""GPU parity of the scaled-MFMA expert path (MXFP8 activations x MXFP4
weights): the MXFP8 quantiser (moe_quantize_mxfp8) bit for bit against the
oracle's, and whole small layers with expert_act_mxfp8 against the oracle
that quantises z and h the same way (tolerance of the MXFP4 layers)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_sigmoid_amd as moe
from synth.configs import LayerConfig

from _gpu_helpers import say, to64, run_layer, check_y

pytestmark = pytest.mark.gpu


def _bf16_rows(rows, K, seed, spread):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, K)) * np.exp2(rng.uniform(-spread, spread, (rows, 1)))
    v[rows // 3] = 0.0                                   # an all-zero row: scale byte 0
    if K >= 64:
        v[0, 5] = 3.0e38                                 # near the bf16 maximum
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    return t, t.float().numpy().astype(np.float64)


@pytest.mark.parametrize("rows,K,spread", [(1, 32, 2), (37, 96, 30), (300, 3584, 120), (5, 4096, 0)])
def test_quantize_mxfp8_bit_exact(rows, K, spread, device):
    say(f"mxfp8 quantise: rows={rows} K={K}")
    x, xv = _bf16_rows(rows, K, seed=rows * 3 + K, spread=spread)
    codes = torch.full((rows, K), 0x5A, dtype=torch.uint8, device=device)
    scales = torch.full((rows, K // 32), 0x5A, dtype=torch.uint8, device=device)
    moe.moe_quantize_mxfp8(x.to(device), codes, scales)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx8_quantize(xv)
    assert np.array_equal(scales.cpu().numpy(), s_ref), "scale bytes differ"
    assert np.array_equal(codes.cpu().numpy(), c_ref), "element codes differ"


def test_quantize_mxfp8_strided_rows(device):
    x, _ = _bf16_rows(20, 256, seed=9, spread=4)
    big = torch.zeros((20, 320), dtype=torch.bfloat16)
    big[:, :256] = x
    xd = big.to(device)[:, :256]                         # row stride 320 elements
    codes = torch.empty((20, 256), dtype=torch.uint8, device=device)
    scales = torch.empty((20, 8), dtype=torch.uint8, device=device)
    moe.moe_quantize_mxfp8(xd, codes, scales)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx8_quantize(x.float().numpy().astype(np.float64))
    assert np.array_equal(codes.cpu().numpy(), c_ref) and np.array_equal(scales.cpu().numpy(), s_ref)


MX8_SMALL = LayerConfig("mx8_small", T=70, d=128, d_lat=128, E=10, k=3, F=256, S=1, Fs=96, seed=41,
                        expert_w="mxfp4", latent_w="mxfp4", expert_act="mxfp8", bias=("uniform", 0.05))
# several 128-row tiles per expert, ragged in rows and in the n-tiles of gate/up and down
MX8_MID = LayerConfig("mx8_mid", T=700, d=256, d_lat=384, E=5, k=2, F=384, S=1, Fs=128, seed=42,
                      expert_w="mxfp4", latent_w="mxfp4", expert_act="mxfp8", bias=("uniform", 0.05))


@pytest.mark.parametrize("cfg", [MX8_SMALL, MX8_MID], ids=lambda c: c.name)
def test_layer_mx8_full_parity(cfg, device):
    say(f"layer {cfg.name}")
    inp = synth.device_inputs(cfg, device)
    y, idx, gate, counts = run_layer(cfg, inp, device)
    y_ref, inter = oracle.forward(cfg, synth.HostWeights(cfg), keep=True)
    assert np.array_equal(idx.cpu().numpy(), inter["idx"])
    assert np.array_equal(gate.cpu().numpy(), inter["p"])
    check_y(cfg, to64(y), y_ref)
    # the scaled path is a different computation: it must not equal the bf16-input path
    y_bf16 = oracle.forward(cfg.replace(expert_act="act"), synth.HostWeights(cfg))
    rms = float(np.sqrt((y_ref ** 2).mean()))
    say(f"  {cfg.name}: MXFP8-input vs bf16-input oracle: max|dy| = "
        f"{np.abs(y_ref - y_bf16).max() / rms:.3e} x RMS")
