"""GPU parity at the K3 layer size for the prefill, skewed-routing and MXFP4
prefill workloads, in the launch configuration bench.py times
(moe_layer_forward, full batch). Routing (indices, gates, counts, and the
permutation of the GPU's own routing) is compared for every token; outputs on
a seeded token sample that includes the hottest and the coldest expert
(tokens are independent in the forward pass, so each sampled row is exact)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_sigmoid_amd as moe

from _gpu_helpers import say, to64, run_layer, check_y, sample_tokens

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,n_sample", [("k3_skew", 10), ("k3_prefill", 8),
                                           ("k3_prefill_mxfp4", 8), ("k3_prefill_mx8", 8),
                                           ("k3_decode_mxfp4", 12), ("k3_decode_mx8", 12)])
def test_k3_full_size(name, n_sample, device):
    cfg = synth.config(name)
    say(f"{name}: generating inputs on the GPU")
    inp = synth.device_inputs(cfg, device)
    y, idx, gate, counts = run_layer(cfg, inp, device)
    idx_np = idx.cpu().numpy()

    # permutation of the GPU routing, on the GPU, vs the oracle's counting sort
    desc = moe.make_desc(cfg)
    T, k, E = cfg.T, cfg.k, cfg.E
    cnt = torch.empty(E, dtype=torch.int32, device=device)
    off = torch.empty(E + 1, dtype=torch.int32, device=device)
    perm = torch.empty(T * k, dtype=torch.int32, device=device)
    inv = torch.empty(T * k, dtype=torch.int32, device=device)
    moe.moe_permute(desc, idx, cnt, off, perm, inv, moe.workspace(desc, moe.MOE_OP_PERMUTE, device))
    torch.cuda.synchronize()

    w = synth.HostWeights(cfg)
    say(f"{name}: oracle routing of all {T} tokens")
    ref = oracle.route_layer(cfg, w)
    assert np.array_equal(idx_np, ref["idx"]), "expert indices differ"
    assert np.array_equal(gate.cpu().numpy(), ref["p"]), "gates differ"
    c_ref, o_ref, p_ref, i_ref = oracle.permute(ref["idx"], E)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(cnt.cpu().numpy(), c_ref)
    assert np.array_equal(off.cpu().numpy(), o_ref)
    assert np.array_equal(perm.cpu().numpy(), p_ref)
    assert np.array_equal(inv.cpu().numpy(), i_ref)
    say(f"{name}: touched {int((c_ref > 0).sum())} experts, max count {int(c_ref.max())}")

    toks = sample_tokens(cfg, idx_np, n_sample)
    say(f"{name}: oracle forward on {len(toks)} tokens")
    y_ref = oracle.forward(cfg, w, tokens=toks,
                           routing={"idx": ref["idx"][toks], "p": ref["p"][toks]})
    check_y(cfg, to64(y)[toks], y_ref, " (sampled tokens)")
