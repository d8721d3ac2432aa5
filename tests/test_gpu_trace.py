"""Stage tracing of the layer (moe_trace_enable / moe_trace_enable_stages):
every stage timed when all are traced, only the selected stage otherwise (the
others read -1), and the trace window resets after each read."""
import pytest
import torch

import synth
import sparse_mixture_experts_sigmoid_amd as moe

pytestmark = pytest.mark.gpu


def test_stage_tracing(device):
    cfg = synth.config("k3_decode")
    inp = moe.prepare_weights(cfg, synth.device_inputs(cfg, device))
    desc = moe.make_desc(cfg)
    ws = moe.workspace(desc, moe.MOE_OP_LAYER, device)
    y = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=device)

    def calls(n):
        for _ in range(n):
            moe.moe_layer_forward(desc, inp, inp["x"], y, None, None, None, ws)
        torch.cuda.synchronize()

    moe.moe_trace_enable(3)
    calls(5)                                   # only the first 3 are traced
    stages, n = moe.moe_trace_read()
    assert n == 3 and len(stages) == moe.MOE_TRACE_STAGES
    assert all(v > 0 for v in stages.values()), stages
    moe.moe_trace_enable(2, stages=["expert_gate_up", "expert_down"])
    calls(2)
    sel, n = moe.moe_trace_read()
    assert n == 2
    assert sel["expert_gate_up"] > 0 and sel["expert_down"] > 0
    assert all(v == -1.0 for k, v in sel.items() if k not in ("expert_gate_up", "expert_down")), sel
    _, n = moe.moe_trace_read()
    assert n == 0                              # the window was reset by the read
    moe.moe_trace_enable(0)
