"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small configs run the oracle on every token; the K3-size decode layer runs the
full routing and a seeded token sample (tokens are independent in the forward
pass, so every sampled row is exact)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_sigmoid_amd as moe
from synth.configs import LayerConfig

from _gpu_helpers import (say, to64, run_layer, check_gates, check_y, sample_tokens, act_torch,
                          staged_front)

pytestmark = pytest.mark.gpu

SMALL_BF16 = LayerConfig("small_bf16", T=70, d=96, d_lat=64, E=10, k=3, F=160, S=2, Fs=96, seed=11,
                         bias=("uniform", 0.05))
SMALL_MX = SMALL_BF16.replace(name="small_mxfp4", expert_w="mxfp4", latent_w="mxfp4", seed=12)
# several 128-row tiles per expert, ragged in M, N and K
MID_BF16 = LayerConfig("mid_bf16", T=700, d=320, d_lat=192, E=6, k=2, F=224, S=1, Fs=160, seed=13,
                       bias=("uniform", 0.05))
MID_MX = MID_BF16.replace(name="mid_mxfp4", expert_w="mxfp4", latent_w="mxfp4", seed=14)
# a batch whose latent-down and output GEMMs run in one pass (at least 256
# tiles of 256 x 256), so the MXFP4 latent maps go through their bf16 copies;
# ragged in M, N and K
WIDE_MX = LayerConfig("wide_mxfp4", T=16300, d=1056, d_lat=992, E=8, k=2, F=256, S=1, Fs=288, seed=15,
                      bias=("uniform", 0.05), expert_w="mxfp4", latent_w="mxfp4")


# ---------------------------------------------------------------------------
# generator twins
# ---------------------------------------------------------------------------

def test_device_generator_matches_host(device):
    cfg = synth.config("k3_decode")
    w = synth.HostWeights(cfg)
    say("generator: bf16 slices")
    for name, row0, rows in (("x", 3, 5), ("W_g", 5 * cfg.F + 7, 33), ("W_os", 100, 3)):
        dt, host = w.raw(name, row0, rows)
        dev = synth.device_tensor(cfg, name, device, row0, rows)
        assert np.array_equal(dev.view(torch.int16).cpu().numpy().view(np.uint16), host), name
    cfg0 = synth.config("tiny_f32")
    dt, host = synth.HostWeights(cfg0).raw("W_v", 40, 17)
    dev = synth.device_tensor(cfg0, "W_v", device, 40, 17)
    assert np.array_equal(dev.cpu().numpy(), host)
    say("generator: mxfp4 slices")
    cfg4 = synth.config("k3_prefill_mxfp4")
    for name, row0, rows in (("W_g", 123 * cfg4.F + 9, 6), ("W_o", 77, 4), ("W_ld", 0, 3)):
        dt, (p, s) = synth.HostWeights(cfg4).raw(name, row0, rows)
        dp, ds = synth.device_tensor(cfg4, name, device, row0, rows)
        assert np.array_equal(dp.cpu().numpy(), p) and np.array_equal(ds.cpu().numpy(), s), name


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

def _route_gpu(cfg, inp, dev, want_scores=True):
    """moe_route with the score output (every logit in fixed order on VALU) or
    without it (bf16: matrix-core logits + exact recheck near the boundary)."""
    desc = moe.make_desc(cfg)
    idx = torch.full((cfg.T, cfg.k), -5, dtype=torch.int32, device=dev)
    gate = torch.full((cfg.T, cfg.k), -5.0, dtype=torch.float32, device=dev)
    s = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev) if want_scores else None
    ws = moe.workspace(desc, moe.MOE_OP_ROUTE, dev)
    moe.moe_route(desc, inp["x"], inp["W_r"], inp["b"], idx, gate, s, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gate.cpu().numpy(), (s.cpu().numpy() if want_scores else None)


ROUTE_CASES = [
    synth.config("tiny_f32"),
    synth.config("k3_decode"),
    LayerConfig("r1", T=1, d=64, d_lat=32, E=5, k=5, F=32, S=0, Fs=32, seed=21),          # k = E
    LayerConfig("r2", T=37, d=96, d_lat=32, E=64, k=1, F=32, S=0, Fs=32, seed=22),
    LayerConfig("r3", T=130, d=160, d_lat=32, E=200, k=70, F=32, S=0, Fs=32, seed=23),    # k > 64
    LayerConfig("r4", T=33, d=64, d_lat=32, E=1, k=1, F=32, S=0, Fs=32, seed=24,
                act="f32", expert_w="f32", latent_w="f32", dense_w="f32"),
    # wide expert counts: 17-32 and 33-64 keys per lane in the recheck, with
    # the register-streamed form (few tokens, d % 256 == 0), the LDS-staged
    # form (d % 256 != 0, or 2048 tokens and more) and k > 64
    LayerConfig("r5", T=70, d=256, d_lat=32, E=1500, k=24, F=32, S=0, Fs=32, seed=27),
    LayerConfig("r6", T=40, d=192, d_lat=32, E=3000, k=100, F=32, S=0, Fs=32, seed=28),
    LayerConfig("r7", T=50, d=512, d_lat=32, E=4000, k=32, F=32, S=0, Fs=32, seed=29),
    LayerConfig("r8", T=2100, d=128, d_lat=32, E=2500, k=16, F=32, S=0, Fs=32, seed=30),
]


@pytest.mark.parametrize("cfg", ROUTE_CASES, ids=lambda c: c.name)
def test_route_bit_exact(cfg, device):
    say(f"route {cfg.name}: T={cfg.T} E={cfg.E} k={cfg.k}")
    inp = {n: synth.device_tensor(cfg, n, device) for n in ("x", "W_r")}
    inp["b"] = torch.from_numpy(synth.bias(cfg)).to(device)
    idx, gate, s = _route_gpu(cfg, inp, device)
    ref = oracle.route_layer(cfg, synth.HostWeights(cfg))
    assert np.array_equal(s, ref["s"]), "sigmoid scores differ"
    assert np.array_equal(idx, ref["idx"]), "expert indices differ"
    check_gates(gate, ref["p"])
    assert np.array_equal(gate, ref["p"])
    say(f"route {cfg.name}: without the score output")
    idx2, gate2, _ = _route_gpu(cfg, inp, device, want_scores=False)
    assert np.array_equal(idx2, ref["idx"]), "expert indices differ (no score output)"
    assert np.array_equal(gate2, ref["p"]), "gates differ (no score output)"


def test_route_ties_go_to_lower_index(device):
    """Duplicate router rows + equal bias -> exactly tied keys."""
    cfg = LayerConfig("ties", T=50, d=64, d_lat=32, E=12, k=4, F=32, S=0, Fs=32, seed=25)
    x = synth.device_tensor(cfg, "x", device)
    W = synth.device_tensor(cfg, "W_r", device).clone()
    W[6:12] = W[0:6]                      # experts e and e+6 tie exactly
    b = torch.zeros(cfg.E, dtype=torch.float32, device=device)
    idx, gate, s = _route_gpu(cfg, {"x": x, "W_r": W, "b": b}, device)
    ref = oracle.route(oracle.widen(("bf16", x.view(torch.int16).cpu().numpy().view(np.uint16))),
                       oracle.widen(("bf16", W.view(torch.int16).cpu().numpy().view(np.uint16))),
                       b.cpu().numpy(), cfg.k)
    assert np.array_equal(s[:, :6], s[:, 6:])
    assert np.array_equal(idx, ref["idx"])
    assert np.array_equal(gate, ref["p"])
    idx2, gate2, _ = _route_gpu(cfg, {"x": x, "W_r": W, "b": b}, device, want_scores=False)
    assert np.array_equal(idx2, ref["idx"])
    assert np.array_equal(gate2, ref["p"])


@pytest.mark.parametrize("shift", [10, 16])
def test_route_near_ties(shift, device):
    """Router rows scaled by 2^-shift (exact in bf16): every logit is tiny, all
    sigmoid scores sit within a few ulp of 1/2 and the keys of most experts tie
    or nearly tie, so the rounding of the logit sums decides the selection.
    With and without the score output the routing must equal the oracle's."""
    cfg = LayerConfig("near_ties", T=96, d=7168, d_lat=32, E=896, k=16, F=32, S=0, Fs=32, seed=26)
    x = synth.device_tensor(cfg, "x", device)
    W = synth.device_tensor(cfg, "W_r", device) * (2.0 ** -shift)
    b = torch.zeros(cfg.E, dtype=torch.float32, device=device)
    ref = oracle.route(oracle.widen(("bf16", x.view(torch.int16).cpu().numpy().view(np.uint16))),
                       oracle.widen(("bf16", W.view(torch.int16).cpu().numpy().view(np.uint16))),
                       b.cpu().numpy(), cfg.k)
    say(f"near ties 2^-{shift}: {len(np.unique(ref['key']))} distinct keys of {ref['key'].size}")
    for want in (True, False):
        idx, gate, _ = _route_gpu(cfg, {"x": x, "W_r": W, "b": b}, device, want_scores=want)
        assert np.array_equal(idx, ref["idx"]), f"indices differ (score output {want})"
        assert np.array_equal(gate, ref["p"]), f"gates differ (score output {want})"


# ---------------------------------------------------------------------------
# permutation
# ---------------------------------------------------------------------------

def _permute_gpu(T, E, k, idx_np, dev):
    cfg = LayerConfig("p", T=T, d=32, d_lat=32, E=E, k=k, F=32, S=0, Fs=32, seed=0)
    desc = moe.make_desc(cfg)
    idx = torch.from_numpy(idx_np.astype(np.int32)).to(dev) if T else torch.empty((0, k), dtype=torch.int32, device=dev)
    counts = torch.full((E,), -7, dtype=torch.int32, device=dev)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    perm = torch.empty((max(T * k, 1),), dtype=torch.int32, device=dev)
    inv = torch.empty((max(T * k, 1),), dtype=torch.int32, device=dev)
    ws = moe.workspace(desc, moe.MOE_OP_PERMUTE, dev)
    moe.moe_permute(desc, idx, counts, offsets, perm, inv, ws)
    torch.cuda.synchronize()
    return (counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy()[:T * k],
            inv.cpu().numpy()[:T * k])


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (63, 7, 3), (64, 7, 7), (65, 896, 16), (1000, 96, 8),
                                   (4096, 896, 16), (300, 4096, 2)])
def test_permute_bit_exact(T, E, k, device):
    rng = np.random.default_rng(T * 7 + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    got = _permute_gpu(T, E, k, idx, device)
    ref = oracle.permute(idx, E)
    for g, r, name in zip(got, ref, ("counts", "offsets", "perm_src", "inv_pos")):
        assert np.array_equal(g, r), name


def test_permute_skewed_and_empty(device):
    # every token on the same 3 experts (others empty), and the empty batch
    T, E, k = 777, 50, 3
    idx = np.tile(np.array([[49, 0, 17]], np.int32), (T, 1))
    got = _permute_gpu(T, E, k, idx, device)
    ref = oracle.permute(idx, E)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    c, o, _, _ = _permute_gpu(0, 9, 2, None, device)
    assert np.all(c == 0) and np.all(o == 0)


# ---------------------------------------------------------------------------
# the whole layer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [synth.config("tiny_f32"), SMALL_BF16, SMALL_MX, MID_BF16, MID_MX],
                         ids=lambda c: c.name)
def test_layer_small_full_parity(cfg, device):
    say(f"layer {cfg.name}")
    inp = synth.device_inputs(cfg, device)
    y, idx, gate, counts = run_layer(cfg, inp, device)
    y_ref, inter = oracle.forward(cfg, synth.HostWeights(cfg), keep=True)
    assert np.array_equal(idx.cpu().numpy(), inter["idx"])
    assert np.array_equal(gate.cpu().numpy(), inter["p"])
    assert np.array_equal(counts.cpu().numpy(), np.bincount(inter["idx"].ravel(), minlength=cfg.E))
    check_y(cfg, to64(y), y_ref)


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_MX,
                                 LayerConfig("small_mx8", T=0, d=128, d_lat=128, E=10, k=3, F=256, S=1,
                                             Fs=96, seed=41, expert_w="mxfp4", latent_w="mxfp4",
                                             expert_act="mxfp8"),
                                 LayerConfig("small_mx8_tiled", T=0, d=128, d_lat=128, E=10, k=3, F=256,
                                             S=1, Fs=96, seed=41, expert_w="mxfp4", latent_w="mxfp4",
                                             expert_act="mxfp8", expert_layout="tiled")],
                         ids=lambda c: c.name)
def test_layer_empty_batch(cfg, device):
    """T = 0: the layer returns MOE_OK without touching token buffers (NULL here,
    as torch gives empty tensors no storage) and reports every expert empty."""
    cfg = cfg.replace(T=0)
    say(f"layer {cfg.name} with T = 0")
    inp = synth.device_inputs(cfg, device)
    y, idx, gate, counts = run_layer(cfg, inp, device)
    assert y.shape == (0, cfg.d) and idx.shape == (0, cfg.k)
    assert counts.cpu().numpy().tolist() == [0] * cfg.E


@pytest.mark.parametrize("cfg", [MID_BF16, WIDE_MX], ids=lambda c: c.name)
def test_staged_entry_points_equal_layer(cfg, device):
    """The staged entry points, each on its own workspace, give the layer's
    routing and output bit for bit (the wide MXFP4 layer: with the latent maps
    decoded to bf16 copies in the latent-down and output workspaces); the mid
    layer's z and u also against the oracle."""
    inp = synth.device_inputs(cfg, device)
    y_layer, idx_l, gate_l, _ = run_layer(cfg, inp, device)
    desc = moe.make_desc(cfg)
    T, k, E = cfg.T, cfg.k, cfg.E
    dt = act_torch(cfg)
    idx = torch.empty((T, k), dtype=torch.int32, device=device)
    gate = torch.empty((T, k), dtype=torch.float32, device=device)
    moe.moe_route(desc, inp["x"], inp["W_r"], inp["b"], idx, gate, None,
                  moe.workspace(desc, moe.MOE_OP_ROUTE, device))
    counts = torch.empty(E, dtype=torch.int32, device=device)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
    perm = torch.empty(T * k, dtype=torch.int32, device=device)
    inv = torch.empty(T * k, dtype=torch.int32, device=device)
    moe.moe_permute(desc, idx, counts, offsets, perm, inv, moe.workspace(desc, moe.MOE_OP_PERMUTE, device))
    z = torch.empty((T, cfg.d_lat), dtype=dt, device=device)
    moe.moe_latent_down(desc, inp["x"], inp["W_ld"], z, moe.workspace(desc, moe.MOE_OP_LATENT_DOWN, device))
    o = torch.empty((T * k, cfg.d_lat), dtype=dt, device=device)
    moe.moe_expert_ffn(desc, z, perm, offsets, inp, o, moe.workspace(desc, moe.MOE_OP_EXPERT_FFN, device))
    n = torch.empty((T, cfg.d_lat), dtype=dt, device=device)
    u = torch.empty((T, cfg.d_lat), dtype=torch.float32, device=device)
    moe.moe_combine(desc, o, inv, gate, inp["gain"], n, u)
    y = torch.empty((T, cfg.d), dtype=dt, device=device)
    moe.moe_output(desc, inp["x"], n, inp, y, moe.workspace(desc, moe.MOE_OP_OUTPUT, device))
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_l) and torch.equal(gate, gate_l)
    assert torch.equal(y, y_layer)
    if cfg.T > 1000:
        return
    # intermediates against the oracle
    y_ref, inter = oracle.forward(cfg, synth.HostWeights(cfg), keep=True)
    z_ref = inter["z"]
    assert np.abs(to64(z) - z_ref).max() <= 2e-2 * np.sqrt((z_ref ** 2).mean())
    u_ref = inter["u"]
    assert np.abs(u.cpu().numpy() - u_ref).max() <= 2e-2 * np.sqrt((u_ref ** 2).mean())


@pytest.mark.parametrize("cfg", [SMALL_MX, MID_MX, WIDE_MX], ids=lambda c: c.name)
def test_mxfp4_path_equals_bf16_path_on_decoded_weights(cfg, device):
    """MXFP4 decoding is exact: the MXFP4 layer must equal, bit for bit, the bf16
    layer run on the decoded weights (same accumulation order). The small layer
    has one row tile per expert, the mid one several, ragged; in the wide one
    the latent maps are decoded to bf16 copies for single-pass dense GEMMs."""
    inp = synth.device_inputs(cfg, device)
    y_mx, _, _, _ = run_layer(cfg, inp, device)
    dec = dict(inp)
    for name in ("W_g", "W_v", "W_o", "W_ld", "W_lu"):
        p, s = inp[name]
        f = oracle.widen(("mxfp4", (p.cpu().numpy(), s.cpu().numpy())))
        dec[name] = torch.from_numpy(f).to(device).to(torch.bfloat16).contiguous()
    cfg_b = cfg.replace(expert_w="bf16", latent_w="bf16")
    y_b, _, _, _ = run_layer(cfg_b, dec, device)
    assert torch.equal(y_mx, y_b)


def test_latent_down_mxfp4_copy_is_exact_for_every_code_and_scale(device):
    """The single-pass latent down of a large batch reads an MXFP4 W_ld through
    its bf16 copy, decoded in the call: for every E2M1 code and every scale byte
    0..200 (scale 2^-127 .. 2^73) z equals, bit for bit, the same GEMM on the
    oracle's decoding of the weight (an OCP E2M1 value times its e8m0 scale is
    exact in bf16 down to 2^-128)."""
    cfg = LayerConfig("latent_mx", T=16384, d=256, d_lat=1024, E=4, k=1, F=64, S=0, Fs=64, seed=21,
                      bias=("uniform", 0.05), expert_w="mxfp4", latent_w="mxfp4")
    cfg_b = cfg.replace(latent_w="bf16")
    desc, desc_b = moe.make_desc(cfg), moe.make_desc(cfg_b)
    # the copy is in use: its d_lat x d bf16 elements are in the workspace
    ws_extra = (moe.moe_workspace_bytes(desc, moe.MOE_OP_LATENT_DOWN) -
                moe.moe_workspace_bytes(desc_b, moe.MOE_OP_LATENT_DOWN))
    assert ws_extra == cfg.d_lat * cfg.d * 2
    g = torch.Generator().manual_seed(21)
    x = torch.randn((cfg.T, cfg.d), generator=g).to(torch.bfloat16).to(device)
    packed = torch.randint(0, 256, (cfg.d_lat, cfg.d // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    scales = (torch.arange(cfg.d_lat * (cfg.d // 32)) % 201).to(torch.uint8).reshape(cfg.d_lat, cfg.d // 32)
    w_b = torch.from_numpy(oracle.widen(("mxfp4", (packed.numpy(), scales.numpy())))).to(torch.bfloat16)
    assert torch.equal(w_b.float(), torch.from_numpy(oracle.widen(("mxfp4", (packed.numpy(), scales.numpy())))))
    z_mx = torch.empty((cfg.T, cfg.d_lat), dtype=torch.bfloat16, device=device)
    z_b = torch.empty_like(z_mx)
    moe.moe_latent_down(desc, x, (packed.to(device), scales.to(device)), z_mx,
                        moe.workspace(desc, moe.MOE_OP_LATENT_DOWN, device))
    moe.moe_latent_down(desc_b, x, w_b.to(device), z_b, moe.workspace(desc_b, moe.MOE_OP_LATENT_DOWN, device))
    torch.cuda.synchronize()
    assert torch.isfinite(z_b.float()).all()
    assert torch.equal(z_mx, z_b)


def test_k3_decode_parity_and_determinism(device):
    cfg = synth.config("k3_decode")
    say("k3_decode: generating inputs on the GPU")
    inp = synth.device_inputs(cfg, device)
    y, idx, gate, counts = run_layer(cfg, inp, device)
    y2, _, _, _ = run_layer(cfg, inp, device)
    assert torch.equal(y, y2), "two runs differ"
    w = synth.HostWeights(cfg)
    say("k3_decode: oracle routing (all tokens)")
    ref = oracle.route_layer(cfg, w)
    idx_np = idx.cpu().numpy()
    assert np.array_equal(idx_np, ref["idx"])
    assert np.array_equal(gate.cpu().numpy(), ref["p"])
    assert np.array_equal(counts.cpu().numpy(), np.bincount(ref["idx"].ravel(), minlength=cfg.E))
    say(f"k3_decode: oracle forward on all {cfg.T} tokens")
    y_ref = oracle.forward(cfg, w, routing={"idx": ref["idx"], "p": ref["p"]})
    check_y(cfg, to64(y), y_ref, " (every token)")


@pytest.mark.parametrize("cfg", [SMALL_BF16, MID_BF16, SMALL_MX, MID_MX], ids=lambda c: c.name)
def test_expert_gate_up_h_against_oracle(cfg, device):
    """Row a5 on its own: moe_expert_gate_up's h (stored bf16, permuted rows)
    against the oracle's h of the same (token, slot), within 2e-2 of RMS(h)
    (5e-2 with MXFP4 weights), on the GPU's own routing and z; and the
    staged gate/up equals the first half of moe_expert_ffn (same o)."""
    say(f"gate/up h: {cfg.name}")
    inp = synth.device_inputs(cfg, device)
    desc, idx, gate, offsets, perm, inv, z = staged_front(cfg, inp, device)
    rows = cfg.T * cfg.k
    h = torch.empty((rows, cfg.F), dtype=torch.bfloat16, device=device)
    moe.moe_expert_gate_up(desc, z, perm, offsets, inp, h=h,
                           ws=moe.workspace(desc, moe.MOE_OP_EXPERT_GATE_UP, device))
    torch.cuda.synchronize()
    y_ref, inter = oracle.forward(cfg, synth.HostWeights(cfg), keep=True)
    assert np.array_equal(idx.cpu().numpy(), inter["idx"])
    p = perm.cpu().numpy().astype(np.int64)
    h_ref = inter["h"].reshape(rows, cfg.F)[p]          # row r holds (t, j) = perm_src[r]
    hg = to64(h)
    rms = float(np.sqrt((h_ref ** 2).mean()))
    err = float(np.abs(hg - h_ref).max())
    tol = 5e-2 if cfg.expert_w == "mxfp4" else 2e-2
    say(f"  {cfg.name}: max|dh| = {err / rms:.3e} x RMS(h) (tol {tol})")
    assert err <= tol * rms
