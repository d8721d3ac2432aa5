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

from _gpu_helpers import say, to64, run_layer, check_y, staged_front

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


def _exhaustive_blocks(amax_bits):
    """Blocks of 32 bf16 values: element 0 is the block maximum (bit pattern
    amax_bits), the other 31 run through every bf16 value of smaller magnitude,
    both signs and both zeros, so every rounding case of one scale is met."""
    amax = np.array([amax_bits << 16], np.uint32).view(np.float32)[0]
    allv = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    cand = allv[np.isfinite(allv) & (np.abs(allv) < amax)]
    n = -(-cand.size // 31)
    body = np.zeros(n * 31, np.float32)
    body[:cand.size] = cand
    blk = np.concatenate([np.full((n, 1), amax, np.float32), body.reshape(n, 31)], axis=1)
    return blk.reshape(-1)


@pytest.mark.parametrize("amax_bits", [0x3FE0, 0x3F80, 0x0C00, 0x0300, 0x7F7F],
                         ids=["1.75", "1.0", "2^-103", "2^-121", "bf16max"])
def test_quantize_mxfp8_every_bf16_value(amax_bits, device):
    """Every bf16 value below the block maximum, at five block scales: a plain
    one, a power of two, a tiny one, one so tiny that X is clamped at -127 and
    bf16 subnormals get nonzero codes, and the bf16 maximum."""
    say(f"mxfp8 quantise: every bf16 value under amax bits {amax_bits:#06x}")
    flat = _exhaustive_blocks(amax_bits)
    K = 32 * 64
    flat = np.concatenate([flat, np.zeros(-flat.size % K, np.float32)])
    x = torch.from_numpy(flat.reshape(-1, K)).to(torch.bfloat16)
    rows = x.shape[0]
    codes = torch.full((rows, K), 0x5A, dtype=torch.uint8, device=device)
    scales = torch.full((rows, K // 32), 0x5A, dtype=torch.uint8, device=device)
    moe.moe_quantize_mxfp8(x.to(device), codes, scales)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx8_quantize(x.float().numpy().astype(np.float64))
    assert np.array_equal(scales.cpu().numpy(), s_ref), "scale bytes differ"
    got = codes.cpu().numpy()
    bad = np.argwhere(got != c_ref)
    assert bad.size == 0, (f"{len(bad)} codes differ, first at {tuple(bad[0])}: "
                           f"v={x[tuple(bad[0])].item()!r} got {got[tuple(bad[0])]:#04x} "
                           f"want {c_ref[tuple(bad[0])]:#04x}")


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
    # the scaled path is a different computation: the GPU output must be much
    # closer to the quantising oracle than to the bf16-input one
    y_bf16 = oracle.forward(cfg.replace(expert_act="act"), synth.HostWeights(cfg))
    rms = float(np.sqrt((y_ref ** 2).mean()))
    e_q = float(np.abs(to64(y) - y_ref).max())
    e_b = float(np.abs(to64(y) - y_bf16).max())
    say(f"  {cfg.name}: MXFP8-input vs bf16-input oracle: max|dy| = "
        f"{np.abs(y_ref - y_bf16).max() / rms:.3e} x RMS; GPU vs them {e_q / rms:.3e}, {e_b / rms:.3e}")
    assert e_b > 3 * e_q, "the GPU output does not follow the MXFP8 quantisation"


@pytest.mark.parametrize("rows,K", [(64, 128), (192, 3584), (1920, 384), (0, 128)])
def test_tile_is_the_documented_permutation(rows, K, device):
    """moe_mxfp4_tile reorders the bytes of an MXFP4 weight as documented,
    bit for bit (numpy reshapes of the same order give the expected values):
    packed byte j of row r's stage kt to ((r/2)(K/128) + kt) 128 + (r%2) 64 + j,
    scale byte (r, b) to ((r/64)(K/128) + b/4) 256 + (r%64) 4 + b%4."""
    rng = np.random.default_rng(rows + K)
    d = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    s = rng.integers(0, 256, (rows, K // 32), dtype=np.uint8)
    dsrc, ssrc = torch.from_numpy(d).to(device), torch.from_numpy(s).to(device)
    dout, sout = torch.full_like(dsrc, 0xAB), torch.full_like(ssrc, 0xAB)
    moe.moe_mxfp4_tile(dsrc, ssrc, dout, sout)
    torch.cuda.synchronize()
    want_d = d.reshape(rows // 2, 2, K // 128, 64).transpose(0, 2, 1, 3).reshape(rows, K // 2)
    want_s = s.reshape(rows // 64, 64, K // 128, 4).transpose(0, 2, 1, 3).reshape(rows, K // 32)
    assert np.array_equal(dout.cpu().numpy(), want_d)
    assert np.array_equal(sout.cpu().numpy(), want_s)


@pytest.mark.parametrize("cfg", [MX8_SMALL, MX8_MID], ids=lambda c: c.name)
def test_layer_mx8_tiled_weights(cfg, device):
    """Tiled expert weights change only where the kernels read the weight and
    scale bytes: the layer output equals, bit for bit, the row-major run's, and
    both meet the oracle."""
    inp = synth.device_inputs(cfg, device)
    y_rows, idx, gate, _ = run_layer(cfg, inp, device)
    cfg_t = cfg.replace(name=cfg.name + "_tiled", expert_layout="tiled")
    y_t, idx_t, gate_t, _ = run_layer(cfg_t, inp, device)
    assert torch.equal(idx, idx_t) and torch.equal(gate, gate_t)
    assert torch.equal(y_rows, y_t)
    y_ref = oracle.forward(cfg, synth.HostWeights(cfg))
    check_y(cfg_t, to64(y_t), y_ref)


@pytest.mark.parametrize("name", ["mx8_small", "mx8_mid", "k3_decode_mx8"])
def test_fused_h_quantisation_equals_quantiser(name, device):
    """The gate/up epilogue that writes h straight in MXFP8 gives, bit for bit,
    the codes and scales of the standalone quantiser (moe_quantize_mxfp8)
    applied to the bf16 h that the same kernel writes without the fusion."""
    cfg = {MX8_SMALL.name: MX8_SMALL, MX8_MID.name: MX8_MID}.get(name) or synth.config(name)
    say(f"fused MXFP8 h: {name}")
    inp = moe.prepare_weights(cfg, synth.device_inputs(cfg, device))
    desc, idx, gate, offsets, perm, inv, z = staged_front(cfg, inp, device)
    rows = cfg.T * cfg.k
    ws = moe.workspace(desc, moe.MOE_OP_EXPERT_GATE_UP, device)
    h = torch.empty((rows, cfg.F), dtype=torch.bfloat16, device=device)
    moe.moe_expert_gate_up(desc, z, perm, offsets, inp, h=h, ws=ws)
    hq = torch.full((rows, cfg.F), 0x5A, dtype=torch.uint8, device=device)
    hqs = torch.full((rows, cfg.F // 32), 0x5A, dtype=torch.uint8, device=device)
    moe.moe_expert_gate_up(desc, z, perm, offsets, inp, hq=hq, hqs=hqs, ws=ws)
    q_ref = torch.empty_like(hq)
    s_ref = torch.empty_like(hqs)
    moe.moe_quantize_mxfp8(h, q_ref, s_ref)
    torch.cuda.synchronize()
    assert torch.equal(hqs, s_ref), "scale bytes differ"
    bad = int((hq != q_ref).sum())
    assert bad == 0, f"{bad} of {hq.numel()} codes differ"
