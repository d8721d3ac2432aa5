"""GPU parity at the K3 layer size for the prefill, skewed-routing and MXFP4
prefill workloads, in the launch configuration bench.py times
(moe_layer_forward, full batch). Routing (indices, gates, counts, and the
permutation of the GPU's own routing) is compared for every token; outputs for
every token of the decode batches and for a seeded sample of 1024 tokens of the
larger batches that includes tokens of the hottest and the coldest expert
(tokens are independent in the forward pass, so each sampled row is exact).
Each layer is also run twice: the two calls must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_sigmoid_amd as moe

from _gpu_helpers import (say, to64, run_layer, check_y, sample_tokens, check_mx8_layer,
                          staged_on_z)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,n_sample", [("k3_skew", 1024), ("k3_prefill", 1024),
                                           ("k3_prefill_mxfp4", 1024), ("k3_prefill_mx8", 1024),
                                           ("k3_decode_mxfp4", 256), ("k3_decode_mx8", 256)])
def test_k3_full_size(name, n_sample, device):
    cfg = synth.config(name)
    say(f"{name}: generating inputs on the GPU")
    inp = synth.device_inputs(cfg, device)
    y, idx, gate, counts = run_layer(cfg, inp, device)
    idx_np = idx.cpu().numpy()
    # a second call on its own workspace gives the same bits (the router's
    # approximate logits may be summed in any order, but they only bound the
    # exact recheck; every other sum on the path has a fixed order)
    y2, idx2, gate2, _ = run_layer(cfg, inp, device)
    assert torch.equal(idx, idx2) and torch.equal(gate, gate2) and torch.equal(y, y2), "two calls differ"
    del y2, idx2, gate2

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
    y_ref, inter = oracle.forward(cfg, w, tokens=toks,
                                  routing={"idx": ref["idx"][toks], "p": ref["p"][toks]}, keep=True)
    if cfg.expert_act != "mxfp8":
        check_y(cfg, to64(y)[toks], y_ref, " (sampled tokens)")
        return
    # MXFP8 expert inputs: the layer's own z (within one bf16 step of the
    # oracle's) decides the z codes; then the staged path on the oracle's z
    inp = moe.prepare_weights(cfg, inp)
    z = torch.empty((T, cfg.d_lat), dtype=torch.bfloat16, device=device)
    moe.moe_latent_down(desc, inp["x"], inp["W_ld"], z, moe.workspace(desc, moe.MOE_OP_LATENT_DOWN, device))
    torch.cuda.synchronize()
    check_mx8_layer(cfg, to64(y)[toks], y_ref, to64(z)[toks], inter["z"], " (sampled tokens, layer)")
    tk = torch.from_numpy(toks).to(device)
    z_ref = torch.from_numpy(inter["z"].astype(np.float32)).to(torch.bfloat16).to(device)
    assert np.array_equal(z_ref.float().cpu().numpy().astype(np.float64), inter["z"])
    y_st, idx_st = staged_on_z(cfg, inp, inp["x"][tk].contiguous(), z_ref, device)
    assert np.array_equal(idx_st.cpu().numpy(), ref["idx"][toks])
    check_y(cfg, to64(y_st), y_ref, " (sampled tokens, staged on the oracle's z)")


@pytest.mark.parametrize("base,T,n_sample", [("k3_decode", 1, 1), ("k3_decode", 5, 5), ("k3_decode", 3000, 256),
                                              ("k3_decode", 5000, 256), ("k3_prefill_mxfp4", 3000, 256)])
def test_k3_batch_sizes_between_the_workloads(base, T, n_sample, device):
    """The K3 bf16 layer at batch sizes between and below the benchmarked ones,
    where the launch choices switch: one and five tokens (split-K dense GEMMs,
    128-row expert tiles, the recheck with rows in registers), 3000 tokens
    (split latent down, single-pass output GEMM: no early shared partials) and
    5000 (every dense GEMM in one pass, 320-row expert tiles); and the MXFP4
    layer at 3000 tokens (latent down reading MXFP4 in split form, output GEMM
    on the per-call bf16 copy of W_up). Routing of every token bit for bit;
    outputs on every token or a seeded sample incl. the hottest and the
    coldest expert's."""
    cfg = synth.config(base).replace(name=f"{base}_T{T}", T=T, seed=40 + T % 7)
    inp = synth.device_inputs(cfg, device)
    y, idx, gate, counts = run_layer(cfg, inp, device)
    w = synth.HostWeights(cfg)
    ref = oracle.route_layer(cfg, w)
    idx_np = idx.cpu().numpy()
    assert np.array_equal(idx_np, ref["idx"]), "expert indices differ"
    assert np.array_equal(gate.cpu().numpy(), ref["p"]), "gates differ"
    assert np.array_equal(counts.cpu().numpy(), np.bincount(ref["idx"].ravel(), minlength=cfg.E))
    toks = sample_tokens(cfg, idx_np, n_sample) if n_sample < T else np.arange(T)
    y_ref = oracle.forward(cfg, w, tokens=toks, routing={"idx": ref["idx"][toks], "p": ref["p"][toks]})
    check_y(cfg, to64(y)[toks], y_ref, f" (T = {T}, {len(toks)} tokens)")
