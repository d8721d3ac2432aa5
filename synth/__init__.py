"""Seeded synthetic inputs for the Stable LatentMoE layer.

The one module that both the CPU checker (``oracle/``) and the GPU feed use.
It holds none of the layer's arithmetic: it maps (seed, tensor id, element
index) to a value with a counter-based generator (see csrc/synth_host.c), so
any slice of any tensor can be regenerated alone. Two twins make the same bits:
the host twin (C, OpenMP) fills numpy arrays; the device twin (HIP) fills GPU
memory in place, so the K3-size weights (~60 GB) never pass through the host.

Input recipe (per LayerConfig):
  x              ~ N(0, 1)                     tensor id 0, [T, d]
  W_r            ~ N(0, 1/d)                   id 1, [E, d]
  b              U(-a, a) or Zipf-shaped        id 2, [E] fp32 (host only)
  W_ld           ~ N(0, 1/d)                   id 3, [d_lat, d]
  W_lu           ~ N(0, 1/d_lat)               id 4, [d, d_lat]
  gain           = 1                           id 5, [d_lat] fp32
  W_g, W_v       ~ N(0, 1/d_lat)               ids 6, 7, [E, F, d_lat]
  W_o            ~ N(0, 1/F)                   id 8, [E, d_lat, F]
  W_g^s, W_v^s   ~ N(0, 1/d)                   ids 9, 10, [S, Fs, d]
  W_o^s          ~ N(0, 1/Fs)                  id 11, [S, d, Fs]
"N(0, s^2)" is the standard normal quantised to 65536 equiprobable bins
(bin-midpoint quantiles, |z| <= 4.17), times s in fp32, then stored in the
tensor's dtype (fp32, bf16 round-to-nearest-even, or OCP MXFP4 from the bf16
master).
"""
from __future__ import annotations

import ctypes
import math
import os
import statistics
from functools import lru_cache

import numpy as np

from .configs import (CONFIGS, LayerConfig, config, TID_X, TID_WR, TID_B, TID_WLD,
                      TID_WLU, TID_GAIN, TID_WG, TID_WV, TID_WO, TID_SWG, TID_SWV,
                      TID_SWO)

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

__all__ = ["CONFIGS", "LayerConfig", "config", "normal_table", "key", "sigma_of",
           "host_normal", "host_mxfp4", "bias", "gain", "HostWeights", "device_inputs",
           "TENSORS"]

# name -> (tensor id, fan_in attribute or None, which weight class)
TENSORS = {
    "x": (TID_X, None, "act"),
    "W_r": (TID_WR, "d", "dense"),
    "W_ld": (TID_WLD, "d", "latent"),
    "W_lu": (TID_WLU, "d_lat", "latent"),
    "W_g": (TID_WG, "d_lat", "expert"),
    "W_v": (TID_WV, "d_lat", "expert"),
    "W_o": (TID_WO, "F", "expert"),
    "W_gs": (TID_SWG, "d", "dense"),
    "W_vs": (TID_SWV, "d", "dense"),
    "W_os": (TID_SWO, "Fs", "dense"),
}


def shape_of(cfg: LayerConfig, name: str):
    c = cfg
    return {
        "x": (c.T, c.d), "W_r": (c.E, c.d), "W_ld": (c.d_lat, c.d), "W_lu": (c.d, c.d_lat),
        "W_g": (c.E, c.F, c.d_lat), "W_v": (c.E, c.F, c.d_lat), "W_o": (c.E, c.d_lat, c.F),
        "W_gs": (c.S, c.Fs, c.d), "W_vs": (c.S, c.Fs, c.d), "W_os": (c.S, c.d, c.Fs),
    }[name]


def dtype_of(cfg: LayerConfig, name: str) -> str:
    cls = TENSORS[name][2]
    return {"act": cfg.act, "dense": cfg.dense_w, "latent": cfg.latent_w,
            "expert": cfg.expert_w}[cls]


@lru_cache(maxsize=None)
def _host():
    if not os.path.exists(HOST_LIB):
        raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(HOST_LIB)
    u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.synth_key.argtypes = [u64, u64]
    lib.synth_key.restype = u64
    lib.synth_normal_f32.argtypes = [u64, u64, i64, f32, vp, vp]
    lib.synth_normal_bf16.argtypes = [u64, u64, i64, f32, vp, vp]
    lib.synth_uniform_f32.argtypes = [u64, u64, i64, f32, vp]
    lib.synth_mxfp4.argtypes = [u64, u64, i64, i64, f32, vp, vp, vp]
    for f in ("synth_normal_f32", "synth_normal_bf16", "synth_uniform_f32", "synth_mxfp4"):
        getattr(lib, f).restype = None
    return lib


@lru_cache(maxsize=None)
def normal_table() -> np.ndarray:
    """fp32 standard-normal quantiles at the midpoints of 65536 equal bins."""
    nd = statistics.NormalDist()
    return np.array([nd.inv_cdf((j + 0.5) / 65536.0) for j in range(65536)], dtype=np.float32)


def key(seed: int, tensor_id: int) -> int:
    return int(_host().synth_key(seed, tensor_id))


def sigma_of(cfg: LayerConfig, name: str) -> float:
    fan = TENSORS[name][1]
    if fan is None:
        return 1.0
    return float(np.float32(1.0 / math.sqrt(getattr(cfg, fan))))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def host_normal(seed: int, tid: int, start: int, n: int, sigma: float, dtype: str) -> np.ndarray:
    """n consecutive elements starting at counter `start`. dtype 'f32' -> float32
    array; 'bf16' -> uint16 array of bf16 bit patterns."""
    tab = normal_table()
    k = key(seed, tid)
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        _host().synth_normal_f32(k, start, n, sigma, _ptr(tab), _ptr(out))
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        _host().synth_normal_bf16(k, start, n, sigma, _ptr(tab), _ptr(out))
    else:
        raise ValueError(dtype)
    return out


def host_mxfp4(seed: int, tid: int, row0: int, rows: int, K: int, sigma: float):
    """(packed uint8 [rows, K/2], scales uint8 [rows, K/32]) for rows row0.. of a
    [*, K] tensor whose bf16 masters are the normal values at counter row*K+k."""
    if K % 32:
        raise ValueError("MXFP4 needs K % 32 == 0")
    packed = np.empty((rows, K // 2), dtype=np.uint8)
    scales = np.empty((rows, K // 32), dtype=np.uint8)
    _host().synth_mxfp4(key(seed, tid), row0, rows, K, sigma, _ptr(normal_table()),
                        _ptr(packed), _ptr(scales))
    return packed, scales


def bias(cfg: LayerConfig) -> np.ndarray:
    """Per-expert selection bias, fp32 [E]."""
    kind = cfg.bias[0]
    if kind == "uniform":
        out = np.empty(cfg.E, dtype=np.float32)
        _host().synth_uniform_f32(key(cfg.seed, TID_B), 0, cfg.E, float(np.float32(cfg.bias[1])),
                                  _ptr(out))
        return out
    if kind == "zipf":
        s, scale = cfg.bias[1], cfg.bias[2]
        rank = np.arange(1, cfg.E + 1, dtype=np.float64)
        b = scale * np.log(rank ** (-s))
        b = b - b.mean()
        return b.astype(np.float32)
    if kind == "zero":
        return np.zeros(cfg.E, dtype=np.float32)
    raise ValueError(kind)


def gain(cfg: LayerConfig) -> np.ndarray:
    return np.ones(cfg.d_lat, dtype=np.float32)


class HostWeights:
    """Host-side access to one config's inputs, any slice regenerated on demand.

    Dense arrays come back as float32 (exact widening of bf16 / MXFP4 storage
    is NOT done here: bf16 tensors come back as uint16 bit patterns and MXFP4
    tensors as (packed, scales) so that the consumer decodes them itself)."""

    def __init__(self, cfg):
        self.cfg = config(cfg)

    def raw(self, name: str, row0: int = 0, rows: int | None = None):
        """Rows [row0, row0+rows) of tensor `name` viewed as 2-D [R, K] (K = last dim).
        Returns ('f32', float32 [rows, K]) | ('bf16', uint16 [rows, K]) |
        ('mxfp4', (packed [rows, K/2], scales [rows, K/32]))."""
        cfg = self.cfg
        shp = shape_of(cfg, name)
        K = shp[-1]
        R = int(np.prod(shp[:-1]))
        if rows is None:
            rows = R - row0
        if row0 < 0 or row0 + rows > R:
            raise IndexError(name)
        tid = TENSORS[name][0]
        sig = sigma_of(cfg, name)
        dt = dtype_of(cfg, name)
        if dt == "mxfp4":
            return "mxfp4", host_mxfp4(cfg.seed, tid, row0, rows, K, sig)
        arr = host_normal(cfg.seed, tid, row0 * K, rows * K, sig, dt).reshape(rows, K)
        return dt, arr

    def bias(self):
        return bias(self.cfg)

    def gain(self):
        return gain(self.cfg)


# ----------------------------------------------------------------------------
# device twin
# ----------------------------------------------------------------------------

@lru_cache(maxsize=None)
def _dev():
    if not os.path.exists(DEV_LIB):
        raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(DEV_LIB)
    u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.synth_dev_normal_f32.argtypes = [u64, u64, i64, f32, vp, vp, vp]
    lib.synth_dev_normal_bf16.argtypes = [u64, u64, i64, f32, vp, vp, vp]
    lib.synth_dev_mxfp4.argtypes = [u64, u64, i64, i64, f32, vp, vp, vp, vp]
    for f in ("synth_dev_normal_f32", "synth_dev_normal_bf16", "synth_dev_mxfp4"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


_dev_tables = {}


def _dev_table(device):
    import torch
    key_ = str(device)
    if key_ not in _dev_tables:
        _dev_tables[key_] = torch.from_numpy(normal_table()).to(device)
    return _dev_tables[key_]


def device_tensor(cfg: LayerConfig, name: str, device="cuda:0", row0: int = 0, rows=None):
    """Generate tensor `name` (or a row range of its 2-D view) straight into GPU
    memory. bf16 -> torch.bfloat16, f32 -> torch.float32, mxfp4 ->
    (packed uint8 [rows, K/2], scales uint8 [rows, K/32])."""
    import torch
    shp = shape_of(cfg, name)
    K = shp[-1]
    R = int(np.prod(shp[:-1]))
    if rows is None:
        rows = R - row0
    tid = TENSORS[name][0]
    sig = sigma_of(cfg, name)
    dt = dtype_of(cfg, name)
    k = key(cfg.seed, tid)
    tab = _dev_table(device)
    stream = torch.cuda.current_stream(device).cuda_stream
    full = (row0 == 0 and rows == R)
    if dt == "mxfp4":
        packed = torch.empty((rows, K // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=device)
        rc = _dev().synth_dev_mxfp4(k, row0, rows, K, sig, tab.data_ptr(), packed.data_ptr(),
                                    scales.data_ptr(), stream)
        if rc:
            raise RuntimeError(f"synth_dev_mxfp4 failed ({rc})")
        if full:
            packed = packed.view(*shp[:-1], K // 2)
            scales = scales.view(*shp[:-1], K // 32)
        return packed, scales
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.empty((rows, K), dtype=tdt, device=device)
    fn = _dev().synth_dev_normal_bf16 if dt == "bf16" else _dev().synth_dev_normal_f32
    rc = fn(k, row0 * K, rows * K, sig, tab.data_ptr(), out.data_ptr(), stream)
    if rc:
        raise RuntimeError(f"synth device generator failed ({rc})")
    return out.view(*shp) if full else out


def device_inputs(cfg, device="cuda:0") -> dict:
    """Every input tensor of the layer, generated on the GPU."""
    import torch
    cfg = config(cfg)
    out = {name: device_tensor(cfg, name, device) for name in TENSORS}
    out["b"] = torch.from_numpy(bias(cfg)).to(device)
    out["gain"] = torch.from_numpy(gain(cfg)).to(device)
    return out
