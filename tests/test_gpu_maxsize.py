"""The largest batch the library takes at the K3 layer shape: the routed
experts gather their z rows through one buffer resource with 32-bit offsets,
so T * d_latent * 2 bytes must stay under 2 GiB, i.e. T <= 299593 tokens
(T + 1 is rejected on the host, tests/test_abi_host.py). At that size the last
token's z row ends 1024 bytes below 2 GiB, the permuted h and o buffers hold
4.8 M rows (29.5 and 34.4 GB), and every 64-bit index path is exercised.

Checked: routing invariants on every token (counts, distinct experts per
token, gates summing to one); routing bit for bit and outputs within the bf16
tolerance against the oracle on a seeded sample of tokens that includes the
first and the last token and tokens of the hottest and the coldest expert."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_sigmoid_amd as moe

from _gpu_helpers import say, to64, run_layer, check_y, sample_tokens

pytestmark = pytest.mark.gpu

T_MAX = ((1 << 31) - 1) // (3584 * 2)


def test_k3_largest_batch(device):
    cfg = synth.config("k3_prefill").replace(name="k3_largest_batch", T=T_MAX, seed=6)
    assert cfg.T * cfg.d_lat * 2 < (1 << 31) <= (cfg.T + 1) * cfg.d_lat * 2
    assert moe.moe_check_desc(moe.make_desc(cfg)) == moe.MOE_OK
    torch.cuda.empty_cache()      # about 145 GB below: weights, x, y and a 74 GB workspace
    say(f"{cfg.name}: T = {cfg.T}, generating inputs on the GPU")
    inp = synth.device_inputs(cfg, device)
    say(f"{cfg.name}: layer forward")
    y, idx, gate, counts = run_layer(cfg, inp, device)
    T, k, E = cfg.T, cfg.k, cfg.E
    idx_np, gate_np, cnt = idx.cpu().numpy(), gate.cpu().numpy(), counts.cpu().numpy()
    assert idx_np.min() >= 0 and idx_np.max() < E
    assert np.array_equal(np.bincount(idx_np.ravel(), minlength=E), cnt)
    assert int(cnt.sum()) == T * k
    srt = np.sort(idx_np, axis=1)
    assert (srt[:, 1:] != srt[:, :-1]).all(), "an expert chosen twice by one token"
    assert (gate_np > 0).all()
    assert np.abs(gate_np.astype(np.float64).sum(1) - 1.0).max() < 1e-5
    say(f"{cfg.name}: touched {int((cnt > 0).sum())} experts, max count {int(cnt.max())}")

    toks = sample_tokens(cfg, idx_np, 64, seed=6)
    assert toks[0] == 0 and toks[-1] == T - 1
    w = synth.HostWeights(cfg)
    say(f"{cfg.name}: oracle routing and forward on {len(toks)} tokens")
    ref = oracle.route_layer(cfg, w, tokens=toks)
    assert np.array_equal(idx_np[toks], ref["idx"]), "expert indices differ"
    assert np.array_equal(gate_np[toks], ref["p"]), "gates differ"
    y_ref = oracle.forward(cfg, w, tokens=toks, routing={"idx": ref["idx"], "p": ref["p"]})
    tk = torch.from_numpy(toks).to(device)
    check_y(cfg, to64(y[tk]), y_ref, " (sampled tokens)")
