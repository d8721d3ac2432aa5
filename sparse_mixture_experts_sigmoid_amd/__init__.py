"""Python binding of libmoe.so, the gfx950 Stable LatentMoE layer (C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch is used for device memory and the current HIP stream. The
entry points keep the C names (moe_route, moe_permute, moe_latent_down,
moe_expert_ffn, moe_combine, moe_output, moe_layer_forward) and take torch
tensors (or None for optional outputs); a non-zero status raises MoeError.

There is no fallback: if libmoe.so is missing, importing the binding's entry
points raises.
"""
from __future__ import annotations

import ctypes
import os
from functools import lru_cache

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the same library (a sanitizer build of
# its host code, say); by default the in-tree libmoe.so
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_MXFP4 = 0, 1, 2
(MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_LATENT_DOWN, MOE_OP_EXPERT_FFN, MOE_OP_COMBINE,
 MOE_OP_OUTPUT, MOE_OP_LAYER, MOE_OP_EXPERT_GATE_UP) = range(8)

DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp4": MOE_MXFP4}

EXPORTS = ["moe_workspace_bytes", "moe_check_desc", "moe_route", "moe_permute", "moe_latent_down",
           "moe_expert_ffn", "moe_expert_gate_up", "moe_combine", "moe_output", "moe_layer_forward",
           "moe_layer_forward_noalloc", "moe_noalloc_scratch_bytes",
           "moe_status_string", "moe_last_error", "moe_trace_enable", "moe_trace_enable_stages",
           "moe_trace_read",
           "moe_trace_stage_name", "moe_qb_bias", "moe_quantize_mxfp8", "moe_mxfp4_tile", "moe_bf16_tile",
           "moe_bf16_tiled_bytes", "moe_mxfp4_frag_tile", "moe_mxfp4_frag_tiled_bytes"]
MOE_TRACE_STAGES = 10


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("situ_c", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("expert_w_dtype", ctypes.c_int32),
                ("latent_w_dtype", ctypes.c_int32), ("dense_w_dtype", ctypes.c_int32),
                ("expert_act_mxfp8", ctypes.c_int32), ("expert_w_tiled", ctypes.c_int32)]


class MoeW(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("router", MoeW), ("router_bias", ctypes.c_void_p),
                ("lat_down", MoeW), ("lat_up", MoeW), ("rms_gain", ctypes.c_void_p),
                ("exp_gate", MoeW), ("exp_up", MoeW), ("exp_down", MoeW),
                ("sh_gate", MoeW), ("sh_up", MoeW), ("sh_down", MoeW)]


@lru_cache(maxsize=None)
def lib():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build()); "
                          "there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    D, W, WS = ctypes.POINTER(MoeDesc), MoeW, ctypes.POINTER(MoeWeights)
    sigs = {
        "moe_workspace_bytes": ([D, i32], sz),
        "moe_check_desc": ([D], i32),
        "moe_route": ([D, vp, W, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_permute": ([D, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_latent_down": ([D, vp, W, vp, vp, sz, vp], i32),
        "moe_expert_ffn": ([D, vp, vp, vp, WS, vp, vp, sz, vp], i32),
        "moe_expert_gate_up": ([D, vp, vp, vp, WS, vp, vp, vp, vp, sz, vp], i32),
        "moe_combine": ([D, vp, vp, vp, vp, vp, vp, vp], i32),
        "moe_output": ([D, vp, vp, WS, vp, vp, sz, vp], i32),
        "moe_layer_forward": ([D, WS, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_layer_forward_noalloc": ([D, WS, vp, vp, vp, vp, vp, vp], i32),
        "moe_noalloc_scratch_bytes": ([], sz),
        "moe_status_string": ([i32], ctypes.c_char_p),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_trace_enable": ([i32], i32),
        "moe_trace_enable_stages": ([i32, ctypes.c_uint], i32),
        "moe_trace_read": ([ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(ctypes.c_int)], i32),
        "moe_trace_stage_name": ([i32], ctypes.c_char_p),
        "moe_qb_bias": ([D, vp, vp, vp, vp], i32),
        "moe_quantize_mxfp8": ([vp, ctypes.c_int64, i32, ctypes.c_int64, vp, vp, vp], i32),
        "moe_mxfp4_tile": ([vp, vp, vp, vp, ctypes.c_int64, i32, vp], i32),
        "moe_bf16_tile": ([vp, vp, ctypes.c_int64, i32, vp], i32),
        "moe_bf16_tiled_bytes": ([ctypes.c_int64, i32], ctypes.c_int64),
        "moe_mxfp4_frag_tile": ([vp, vp, vp, vp, ctypes.c_int64, i32, vp], i32),
        "moe_mxfp4_frag_tiled_bytes": ([ctypes.c_int64, i32, ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_int64)], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def make_desc(cfg, T=None) -> MoeDesc:
    """Descriptor from any object with T, d, d_lat, E, k, F, S, Fs, c, eps and the
    dtype names act, expert_w, latent_w, dense_w ('f32' | 'bf16' | 'mxfp4')."""
    return MoeDesc(T=cfg.T if T is None else T, d_model=cfg.d, d_latent=cfg.d_lat,
                   n_experts=cfg.E, top_k=cfg.k, d_ff=cfg.F, n_shared=cfg.S, d_ff_shared=cfg.Fs,
                   situ_c=cfg.c, rms_eps=cfg.eps, act_dtype=DTYPES[cfg.act],
                   expert_w_dtype=DTYPES[cfg.expert_w], latent_w_dtype=DTYPES[cfg.latent_w],
                   dense_w_dtype=DTYPES[cfg.dense_w],
                   expert_act_mxfp8=1 if getattr(cfg, "expert_act", "act") == "mxfp8" else 0,
                   expert_w_tiled=1 if getattr(cfg, "expert_layout", "rows") == "tiled" else 0)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def make_w(t) -> MoeW:
    """bf16 / fp32 tensor -> MoeW(data); (packed, scales) pair -> MoeW(data, scale)."""
    if t is None:
        return MoeW(None, None)
    if isinstance(t, (tuple, list)):
        return MoeW(_ptr(t[0]), _ptr(t[1]))
    return MoeW(_ptr(t), None)


def make_weights(w: dict) -> MoeWeights:
    """Keys: W_r, b, W_ld, W_lu, gain (optional), W_g, W_v, W_o, W_gs, W_vs, W_os."""
    return MoeWeights(router=make_w(w.get("W_r")), router_bias=_ptr(w.get("b")),
                      lat_down=make_w(w.get("W_ld")), lat_up=make_w(w.get("W_lu")),
                      rms_gain=_ptr(w.get("gain")),
                      exp_gate=make_w(w.get("W_g")), exp_up=make_w(w.get("W_v")),
                      exp_down=make_w(w.get("W_o")),
                      sh_gate=make_w(w.get("W_gs")), sh_up=make_w(w.get("W_vs")),
                      sh_down=make_w(w.get("W_os")))


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int):
    if status != MOE_OK:
        msg = lib().moe_last_error().decode() or lib().moe_status_string(status).decode()
        raise MoeError(status, msg)


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------

def moe_check_desc(desc: MoeDesc) -> int:
    return lib().moe_check_desc(ctypes.byref(desc))


def moe_workspace_bytes(desc: MoeDesc, op: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(desc), op))


def moe_route(desc, x, router, bias, topk_idx, topk_gate, scores=None, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_route(ctypes.byref(desc), _ptr(x), make_w(router), _ptr(bias), _ptr(topk_idx),
                           _ptr(topk_gate), _ptr(scores), p, n, _stream(stream)))


def moe_permute(desc, topk_idx, counts, offsets, perm_src, inv_pos, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_permute(ctypes.byref(desc), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                             _ptr(perm_src), _ptr(inv_pos), p, n, _stream(stream)))


def moe_latent_down(desc, x, lat_down, z, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_latent_down(ctypes.byref(desc), _ptr(x), make_w(lat_down), _ptr(z), p, n,
                                 _stream(stream)))


def moe_expert_ffn(desc, z, perm_src, offsets, weights: dict, o_perm, ws=None, stream=None):
    p, n = _ws(ws)
    w = make_weights(weights)
    _check(lib().moe_expert_ffn(ctypes.byref(desc), _ptr(z), _ptr(perm_src), _ptr(offsets),
                                ctypes.byref(w), _ptr(o_perm), p, n, _stream(stream)))


def moe_expert_gate_up(desc, z, perm_src, offsets, weights: dict, h=None, hq=None, hqs=None,
                       ws=None, stream=None):
    """h [T*k, F] in the act dtype, or (expert_act_mxfp8 only) hq [T*k, F] and
    hqs [T*k, F/32] uint8: give one of the two."""
    p, n = _ws(ws)
    w = make_weights(weights)
    _check(lib().moe_expert_gate_up(ctypes.byref(desc), _ptr(z), _ptr(perm_src), _ptr(offsets),
                                    ctypes.byref(w), _ptr(h), _ptr(hq), _ptr(hqs), p, n,
                                    _stream(stream)))


def moe_combine(desc, o_perm, inv_pos, topk_gate, rms_gain, n_out, u_out=None, stream=None):
    _check(lib().moe_combine(ctypes.byref(desc), _ptr(o_perm), _ptr(inv_pos), _ptr(topk_gate),
                             _ptr(rms_gain), _ptr(n_out), _ptr(u_out), _stream(stream)))


def moe_output(desc, x, n, weights: dict, y, ws=None, stream=None):
    p, nb = _ws(ws)
    w = make_weights(weights)
    _check(lib().moe_output(ctypes.byref(desc), _ptr(x), _ptr(n), ctypes.byref(w), _ptr(y), p, nb,
                            _stream(stream)))


def moe_layer_forward(desc, weights: dict, x, y, topk_idx=None, topk_gate=None, counts=None,
                      ws=None, stream=None):
    p, n = _ws(ws)
    w = make_weights(weights)
    _check(lib().moe_layer_forward(ctypes.byref(desc), ctypes.byref(w), _ptr(x), _ptr(y),
                                   _ptr(topk_idx), _ptr(topk_gate), _ptr(counts), p, n,
                                   _stream(stream)))


def moe_layer_forward_noalloc(desc, weights: dict, x, y, topk_idx=None, topk_gate=None,
                              counts=None, stream=None):
    """moe_layer_forward on the library's fixed scratch (no workspace argument)."""
    w = make_weights(weights)
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(desc), ctypes.byref(w), _ptr(x), _ptr(y),
                                           _ptr(topk_idx), _ptr(topk_gate), _ptr(counts),
                                           _stream(stream)))


def moe_noalloc_scratch_bytes() -> int:
    return int(lib().moe_noalloc_scratch_bytes())


def moe_qb_bias(desc, scores, bias_out, quantile_out, stream=None):
    """Quantile Balancing bias from router scores [T, E] (fp32 device tensors)."""
    _check(lib().moe_qb_bias(ctypes.byref(desc), _ptr(scores), _ptr(bias_out), _ptr(quantile_out),
                             _stream(stream)))


def moe_quantize_mxfp8(x, codes, scales, stream=None):
    """MXFP8 codes [rows, K] uint8 and e8m0 scales [rows, K/32] of bf16 rows x [rows, K]."""
    rows, K = x.shape
    _check(lib().moe_quantize_mxfp8(_ptr(x), rows, K, x.stride(0), _ptr(codes), _ptr(scales),
                                    _stream(stream)))


def moe_mxfp4_tile(data, scale, data_out, scale_out, stream=None):
    """Tiled copy (data_out, scale_out) of a row-major MXFP4 weight: packed
    [rows, K/2] and scales [rows, K/32], uint8 device tensors."""
    rows, kb = scale.shape
    _check(lib().moe_mxfp4_tile(_ptr(data), _ptr(scale), _ptr(data_out), _ptr(scale_out), rows,
                                kb * 32, _stream(stream)))


def moe_bf16_tile(data, data_out, stream=None):
    """Fragment-tiled copy of a bf16 weight [rows, K] into data_out (a device
    byte tensor of moe_bf16_tiled_bytes(rows, K) bytes)."""
    rows, K = data.shape
    _check(lib().moe_bf16_tile(_ptr(data), _ptr(data_out), rows, K, _stream(stream)))


def moe_bf16_tiled_bytes(rows: int, K: int) -> int:
    return int(lib().moe_bf16_tiled_bytes(rows, K))


def moe_mxfp4_frag_tiled_bytes(rows: int, K: int) -> tuple[int, int]:
    """(packed bytes, scale bytes) of the fragment-tiled copy of an MXFP4 weight."""
    d, s = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().moe_mxfp4_frag_tiled_bytes(rows, K, ctypes.byref(d), ctypes.byref(s)))
    return int(d.value), int(s.value)


def moe_mxfp4_frag_tile(data, scale, data_out, scale_out, stream=None):
    """Fragment-tiled copy (data_out, scale_out) of a row-major MXFP4 weight:
    packed [rows, K/2] and scales [rows, K/32], uint8 device tensors."""
    rows, kb = scale.shape
    _check(lib().moe_mxfp4_frag_tile(_ptr(data), _ptr(scale), _ptr(data_out), _ptr(scale_out), rows,
                                     kb * 32, _stream(stream)))


def prepare_weights(cfg, weights: dict, stream=None) -> dict:
    """The weight dict the layer reads for `cfg`: the same tensors, except that a
    config with expert_layout == 'tiled' gets tiled copies of W_g, W_v and W_o
    (made once here, on the device, not per batch): the MXFP4 tiled layout for
    MXFP4 expert weights, the fragment-tiled layout for bf16 ones."""
    if getattr(cfg, "expert_layout", "rows") != "tiled":
        return weights
    import torch
    out = dict(weights)
    if getattr(cfg, "expert_w", "bf16") == "bf16":
        for name in ("W_g", "W_v", "W_o"):
            w = weights[name]
            w2 = w.reshape(-1, w.shape[-1])
            t = torch.empty(moe_bf16_tiled_bytes(w2.shape[0], w2.shape[1]), dtype=torch.uint8,
                            device=w.device)
            moe_bf16_tile(w2, t, stream)
            out[name] = t
        return out
    if getattr(cfg, "expert_act", "act") != "mxfp8":
        for name in ("W_g", "W_v", "W_o"):
            packed, scale = weights[name]
            p2, s2 = packed.reshape(-1, packed.shape[-1]), scale.reshape(-1, scale.shape[-1])
            nd, ns = moe_mxfp4_frag_tiled_bytes(p2.shape[0], s2.shape[1] * 32)
            tp = torch.empty(nd, dtype=torch.uint8, device=packed.device)
            ts = torch.empty(ns, dtype=torch.uint8, device=packed.device)
            moe_mxfp4_frag_tile(p2, s2, tp, ts, stream)
            out[name] = (tp, ts)
        return out
    for name in ("W_g", "W_v", "W_o"):
        packed, scale = weights[name]
        p2, s2 = packed.reshape(-1, packed.shape[-1]), scale.reshape(-1, scale.shape[-1])
        tp, ts = torch.empty_like(p2), torch.empty_like(s2)
        moe_mxfp4_tile(p2, s2, tp, ts, stream)
        out[name] = (tp.view(packed.shape), ts.view(scale.shape))
    return out


def moe_trace_enable(max_calls: int, stages=None):
    """Trace the next max_calls layer calls: every stage, or only the named ones."""
    if stages is None:
        _check(lib().moe_trace_enable(max_calls))
        return
    names = [lib().moe_trace_stage_name(i).decode() for i in range(MOE_TRACE_STAGES)]
    mask = 0
    for st in stages:
        mask |= 1 << names.index(st)
    _check(lib().moe_trace_enable_stages(max_calls, mask))


def moe_trace_read() -> tuple[dict, int]:
    """({stage name: average ms}, number of traced calls) of the current window."""
    ms = (ctypes.c_float * MOE_TRACE_STAGES)()
    n = ctypes.c_int(0)
    _check(lib().moe_trace_read(ms, MOE_TRACE_STAGES, ctypes.byref(n)))
    names = [lib().moe_trace_stage_name(i).decode() for i in range(MOE_TRACE_STAGES)]
    return dict(zip(names, [float(v) for v in ms])), int(n.value)


def workspace(desc: MoeDesc, op: int, device="cuda:0"):
    """A device byte tensor of moe_workspace_bytes(desc, op) bytes (at least 1)."""
    import torch
    return torch.empty(max(moe_workspace_bytes(desc, op), 1), dtype=torch.uint8, device=device)
