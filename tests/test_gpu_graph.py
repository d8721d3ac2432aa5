"""The layer captured into a HIP graph (torch.cuda.CUDAGraph over the
library's stream) and replayed: both the workspace entry point and the
allocation-free one (moe_layer_forward_noalloc) are recorded once after an
eager warm-up call (which creates the per-device side stream and resolves the
scratch address), then replayed three times with eager layer calls and
synchronisations between the replays; every replay must give, bit for bit,
the eager result (routing, gates, counts and y)."""
import pytest
import torch

import synth
import sparse_mixture_experts_sigmoid_amd as moe

from _gpu_helpers import say, run_layer

pytestmark = pytest.mark.gpu


def _outputs(cfg, dev):
    return (torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=dev),
            torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev),
            torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev),
            torch.empty((cfg.E,), dtype=torch.int32, device=dev))


def _poison(out):
    y, idx, gate, counts = out
    y.fill_(float("nan"))
    idx.fill_(-7)
    gate.fill_(-1.0)
    counts.fill_(-7)


@pytest.mark.parametrize("name", ["k3_decode", "k3_decode_mx8"])
@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_layer_replays_from_a_graph(entry, name, device):
    cfg = synth.config(name)
    raw = synth.device_inputs(cfg, device)
    inp = moe.prepare_weights(cfg, raw)
    desc = moe.make_desc(cfg)
    y0, i0, g0, c0 = run_layer(cfg, raw, device)
    ws = moe.workspace(desc, moe.MOE_OP_LAYER, device) if entry == "workspace" else None

    def call(out):
        y, idx, gate, counts = out
        if entry == "workspace":
            moe.moe_layer_forward(desc, inp, raw["x"], y, idx, gate, counts, ws)
        else:
            moe.moe_layer_forward_noalloc(desc, inp, raw["x"], y, idx, gate, counts)

    out = _outputs(cfg, device)
    call(out)                                    # warm-up: side stream, scratch address
    torch.cuda.synchronize()
    _poison(out)
    torch.cuda.synchronize()
    say(f"graph: capturing the {entry} layer ({cfg.name})")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    torch.cuda.synchronize()
    other = _outputs(cfg, device)
    for rep in range(3):
        _poison(out)
        call(other)                              # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y, idx, gate, counts = out
        assert torch.equal(idx, i0), f"replay {rep}: expert indices differ"
        assert torch.equal(gate, g0), f"replay {rep}: gates differ"
        assert torch.equal(counts, c0), f"replay {rep}: counts differ"
        assert torch.equal(y, y0), f"replay {rep}: y differs"
        assert torch.equal(other[0], y0), f"eager call between replays {rep}: y differs"
    say(f"graph: {entry} layer, 3 replays bit-identical to the eager call")
