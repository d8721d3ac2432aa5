"""Fragment-tiled expert weights (expert_w_tiled with bf16 activations): the
tilers reorder bytes exactly as documented in include/moe.h (checked against
numpy reshapes of the same order), and the layer on tiled weights equals, bit
for bit, the layer on the row-major weights: the expert kernels that keep the
weights in registers take the same values in the same accumulation order."""
import numpy as np
import pytest
import torch

import synth
import sparse_mixture_experts_sigmoid_amd as moe
from synth.configs import LayerConfig

from _gpu_helpers import say, run_layer

pytestmark = pytest.mark.gpu

SMALL_BF16 = LayerConfig("small_bf16", T=70, d=96, d_lat=64, E=10, k=3, F=160, S=2, Fs=96, seed=11,
                         bias=("uniform", 0.05))
MID_BF16 = LayerConfig("mid_bf16", T=700, d=320, d_lat=192, E=6, k=2, F=224, S=1, Fs=160, seed=13,
                       bias=("uniform", 0.05))
SMALL_MX = SMALL_BF16.replace(name="small_mxfp4", expert_w="mxfp4", latent_w="mxfp4", seed=12)
MID_MX = MID_BF16.replace(name="mid_mxfp4", expert_w="mxfp4", latent_w="mxfp4", seed=14)


@pytest.mark.parametrize("rows,K", [(32, 64), (96, 200), (64, 3584), (0, 64)])
def test_bf16_tile_is_the_documented_order(rows, K, device):
    rng = np.random.default_rng(rows + K)
    w = rng.integers(0, 1 << 16, (rows, K), dtype=np.uint16)
    src = torch.from_numpy(w.view(np.int16)).to(device)
    out = torch.full((moe.moe_bf16_tiled_bytes(rows, K) if rows else 16,), 0xAB, dtype=torch.uint8,
                     device=device)
    if rows:
        moe.moe_bf16_tile(src.view(torch.bfloat16), out)
    torch.cuda.synchronize()
    if rows == 0:
        return
    Kp = -(-K // 64) * 64
    wp = np.zeros((rows, Kp), np.uint16)
    wp[:, :K] = w
    # [g][s][lane: h = l/32, r = l%32][8]: row 32 g + r, k = 16 s + 8 h + e
    want = wp.reshape(rows // 32, 32, Kp // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("rows,K", [(32, 128), (64, 96), (96, 3584), (0, 64)])
def test_mxfp4_frag_tile_is_the_documented_order(rows, K, device):
    rng = np.random.default_rng(rows * 7 + K)
    d = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    s = rng.integers(0, 256, (rows, K // 32), dtype=np.uint8)
    if rows == 0:
        assert moe.lib().moe_mxfp4_frag_tile(None, None, None, None, 0, K, None) == moe.MOE_OK
        return
    nd, ns = moe.moe_mxfp4_frag_tiled_bytes(rows, K)
    dout = torch.full((nd,), 0xAB, dtype=torch.uint8, device=device)
    sout = torch.full((ns,), 0xAB, dtype=torch.uint8, device=device)
    moe.moe_mxfp4_frag_tile(torch.from_numpy(d).to(device), torch.from_numpy(s).to(device), dout, sout)
    torch.cuda.synchronize()
    Kp = -(-K // 128) * 128
    dp = np.zeros((rows, Kp // 2), np.uint8)
    dp[:, :K // 2] = d
    sp = np.zeros((rows, Kp // 32), np.uint8)
    sp[:, :K // 32] = s
    # codes: [g][t][lane: h, r][s][4 bytes]: row 32 g + r, bytes of k = 64 t + 16 s + 8 h .. +7
    want_d = dp.reshape(rows // 32, 32, Kp // 64, 4, 2, 4).transpose(0, 2, 4, 1, 3, 5).reshape(-1)
    # scales: [g][pair][r][4]
    want_s = sp.reshape(rows // 32, 32, Kp // 128, 4).transpose(0, 2, 1, 3).reshape(-1)
    assert np.array_equal(dout.cpu().numpy(), want_d)
    assert np.array_equal(sout.cpu().numpy(), want_s)


@pytest.mark.parametrize("cfg", [SMALL_BF16, MID_BF16, SMALL_MX, MID_MX,
                                 synth.config("k3_decode_mxfp4").replace(expert_layout="rows")],
                         ids=lambda c: c.name)
def test_tiled_layer_equals_row_major_layer(cfg, device):
    say(f"tiled experts: {cfg.name}")
    inp = synth.device_inputs(cfg, device)
    y_rows, idx, gate, counts = run_layer(cfg, inp, device)
    cfg_t = cfg.replace(name=cfg.name + "_tiled", expert_layout="tiled")
    y_t, idx_t, gate_t, counts_t = run_layer(cfg_t, inp, device)
    assert torch.equal(idx, idx_t) and torch.equal(gate, gate_t) and torch.equal(counts, counts_t)
    assert torch.equal(y_rows, y_t), "tiled-weight layer differs from the row-major one"
