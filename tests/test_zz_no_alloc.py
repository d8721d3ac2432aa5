"""The allocation-free layer entry point (moe_layer_forward_noalloc) against
moe_layer_forward: the same kernels on the same inputs give the same bits
(routing, gates, counts and y), on two calls in a row, the second with a
smaller batch; a batch beyond the fixed scratch is rejected on the host."""
import ctypes

import pytest
import torch

import synth
import sparse_mixture_experts_sigmoid_amd as moe

from _gpu_helpers import say, run_layer

pytestmark = pytest.mark.gpu


def _noalloc(cfg, inp, x, dev):
    desc = moe.make_desc(cfg)
    y = torch.full((cfg.T, cfg.d), float("nan"), dtype=torch.bfloat16, device=dev)
    idx = torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, device=dev)
    gate = torch.full((cfg.T, cfg.k), -1.0, dtype=torch.float32, device=dev)
    counts = torch.full((cfg.E,), -7, dtype=torch.int32, device=dev)
    moe.moe_layer_forward_noalloc(desc, inp, x, y, idx, gate, counts)
    torch.cuda.synchronize()
    return y, idx, gate, counts


@pytest.mark.parametrize("name", ["k3_decode", "k3_decode_mx8"])
def test_noalloc_equals_layer_forward_twice(name, device):
    cfg = synth.config(name)
    say(f"noalloc: {name}, T = {cfg.T} then 100 tokens")
    raw = synth.device_inputs(cfg, device)
    inp = moe.prepare_weights(cfg, raw)          # run_layer prepares its own copy from raw
    assert moe.moe_workspace_bytes(moe.make_desc(cfg), moe.MOE_OP_LAYER) <= moe.moe_noalloc_scratch_bytes()
    for T in (cfg.T, 100):
        c = cfg.replace(T=T)
        x = raw["x"][:T].contiguous()
        y_ref, idx_ref, gate_ref, counts_ref = run_layer(c, dict(raw, x=x), device)
        y, idx, gate, counts = _noalloc(c, inp, x, device)
        assert torch.equal(idx, idx_ref), f"T={T}: expert indices differ"
        assert torch.equal(gate, gate_ref), f"T={T}: gates differ"
        assert torch.equal(counts, counts_ref), f"T={T}: counts differ"
        assert torch.equal(y, y_ref), f"T={T}: y differs"


def test_noalloc_rejects_a_batch_beyond_its_scratch(device):
    cfg = synth.config("k3_decode").replace(T=2048)
    desc = moe.make_desc(cfg)
    assert moe.moe_workspace_bytes(desc, moe.MOE_OP_LAYER) > moe.moe_noalloc_scratch_bytes()
    fake = 0x7f0000001000
    w = moe.make_weights({k: fake for k in ("W_r", "b", "W_ld", "W_lu", "W_g", "W_v", "W_o",
                                           "W_gs", "W_vs", "W_os")})
    st = moe.lib().moe_layer_forward_noalloc(ctypes.byref(desc), ctypes.byref(w), fake, fake,
                                             None, None, None, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
    assert b"scratch" in moe.lib().moe_last_error()
