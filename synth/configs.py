"""Workload descriptions of the Stable LatentMoE layer (shapes, dtypes, seeds,
input distributions). Pure data: no arithmetic of the layer lives here.

Shapes of the K3-size layer follow the Kimi K3 numbers table on
"Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか"
(lilting.ch, section "K3のエキスパートは896個の小型LLMではない", the K3 table):
hidden 7168, 896 routed experts, top-16, 2 shared experts, latent 3584,
expert intermediate 3072. The shared-expert intermediate (3072), the SiTU-GLU
cap c = 8 and the tiny fp32 layer are part of the workload specification, not
of the pages.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

# tensor ids of the counter-based generator (one id per logical tensor; an
# expert's slice of W_g / W_v / W_o is a contiguous counter range)
TID_X, TID_WR, TID_B, TID_WLD, TID_WLU, TID_GAIN = 0, 1, 2, 3, 4, 5
TID_WG, TID_WV, TID_WO = 6, 7, 8
TID_SWG, TID_SWV, TID_SWO = 9, 10, 11


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens
    d: int            # d_model
    d_lat: int        # latent width seen by the routed experts
    E: int            # routed experts
    k: int            # experts per token
    F: int            # routed expert intermediate
    S: int            # shared experts
    Fs: int           # shared expert intermediate
    seed: int
    act: str = "bf16"          # activations: "f32" | "bf16"
    expert_w: str = "bf16"     # routed expert weights: "f32" | "bf16" | "mxfp4"
    latent_w: str = "bf16"     # W_down / W_up of the latent maps
    dense_w: str = "bf16"      # router and shared experts
    expert_act: str = "act"    # routed experts' GEMM inputs: "act" (act dtype) | "mxfp8"
    expert_layout: str = "rows"  # expert weight layout in HBM: "rows" | "tiled" (made at load)
    bias: tuple = ("uniform", 0.05)   # ("uniform", halfwidth) | ("zipf", s, scale)
    c: float = 8.0             # SiTU-GLU cap
    eps: float = 1e-6          # RMSNorm epsilon

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def flops_per_token(self) -> int:
        """Algorithmic multiply-adds x2 of one token through the layer."""
        router = 2 * self.d * self.E
        latent = 2 * self.d * self.d_lat * 2
        experts = self.k * (2 * 2 * self.d_lat * self.F + 2 * self.F * self.d_lat)
        shared = self.S * (2 * 2 * self.d * self.Fs + 2 * self.Fs * self.d)
        return router + latent + experts + shared


K3 = dict(d=7168, d_lat=3584, E=896, k=16, F=3072, S=2, Fs=3072)

CONFIGS = [
    LayerConfig("tiny_f32", T=64, d=256, d_lat=128, E=32, k=4, F=96, S=1, Fs=192, seed=0,
                act="f32", expert_w="f32", latent_w="f32", dense_w="f32",
                bias=("uniform", 0.1)),
    LayerConfig("k3_decode", T=256, seed=1, bias=("uniform", 0.05), **K3),
    LayerConfig("k3_prefill", T=16384, seed=2, bias=("uniform", 0.05), **K3),
    # Zipf-shaped selection bias: b_e = 0.5 * ln(rank_e ** -1.1), rank_e = e + 1,
    # shifted to zero mean (computed in fp64, stored fp32)
    LayerConfig("k3_skew", T=8192, seed=3, bias=("zipf", 1.1, 0.5), **K3),
    # MXFP4 expert weights are re-laid once at load into the fragment order
    # (expert_layout "tiled": loaded straight into registers, decoded there)
    LayerConfig("k3_prefill_mxfp4", T=16384, seed=4, expert_w="mxfp4", latent_w="mxfp4",
                expert_layout="tiled", bias=("uniform", 0.05), **K3),
    # the MXFP4 prefill layer with its routed experts on the scaled MFMA
    # (z and h quantised to MXFP8, expert weights tiled once at load);
    # same inputs as k3_prefill_mxfp4
    LayerConfig("k3_prefill_mx8", T=16384, seed=4, expert_w="mxfp4", latent_w="mxfp4",
                expert_act="mxfp8", expert_layout="tiled", bias=("uniform", 0.05), **K3),
    # the decode batch with the deployment weight format: MXFP4 expert and
    # latent weights, decoded to bf16 in the GEMM (..._mxfp4) or fed to the
    # scaled MFMA with MXFP8 expert inputs (..._mx8); same inputs as k3_decode
    LayerConfig("k3_decode_mxfp4", T=256, seed=1, expert_w="mxfp4", latent_w="mxfp4",
                expert_layout="tiled", bias=("uniform", 0.05), **K3),
    LayerConfig("k3_decode_mx8", T=256, seed=1, expert_w="mxfp4", latent_w="mxfp4",
                expert_act="mxfp8", expert_layout="tiled", bias=("uniform", 0.05), **K3),
]

BY_NAME = {c.name: c for c in CONFIGS}


def config(ref) -> LayerConfig:
    if isinstance(ref, LayerConfig):
        return ref
    if isinstance(ref, int):
        return CONFIGS[ref]
    return BY_NAME[ref]
