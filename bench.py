#!/usr/bin/env python3
"""Throughput of the Stable LatentMoE layer forward on one MI355X.

One step = one moe_layer_forward call (router, top-k + gates, permutation,
latent down, routed experts, combine + RMSNorm, shared experts, latent up) on
one batch of seeded synthetic inputs already resident in HBM. Prints ONE JSON
line.

Headline workload: the K3-shape prefill layer (T = 16384 tokens, d = 7168,
d_lat = 3584, 896 experts, top-16, F = 3072, 2 shared experts with Fs = 3072,
bf16 weights and activations, fp32 accumulation), priced against the bf16
matrix-core peak. The decode layer (T = 256, priced against HBM bandwidth on
the touched experts' weights), the skewed-routing layer, the MXFP4-weight
layers and the scaled-MFMA (MXFP8 x MXFP4) layers follow in the same run under
"workloads", each with its own roofline and CPU baseline (--extra).

roofline: the dominant kernel's algorithmic rate from HIP events recorded by
the library around every stage of the timed calls (moe_trace_*), on the stream
the kernels run on. Decode (T <= 1024): the expert gate/up grouped GEMM is
HBM-bound; its algorithmic bytes per launch = (touched experts) x 2*F*d_lat*w B
(W_g and W_v; w = 2 for bf16, 17/32 for MXFP4 with its scales) + (T*k routed
rows) x (z row in + h row out: d_lat*2 + F*2 B, or (d_lat + F)*33/32 B in
MXFP8). Prefill: the same kernel is MFMA-bound; flops per launch =
T*k*2*2*d_lat*F. `peak` is the published MI355X figure; `measured_peak` the
ceiling probed on this GPU in the same run (`ceilings`).

roofline.traffic: HBM bytes per launch of that kernel from rocprofv3 PMC
counters (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for
a plain copy of known size), as recorded in profiles/hbm_traffic.md together
with the hash of the GEMM source they were taken on; null when that source has
changed since.

cpu_baseline: the CPU oracle (never tuned) on a bounded token sample of the
same workload, on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix (the scaled MXFP8 x MXFP4 expert path)
VALU_FP32_PEAK_TFLOPS = 157.3   # MI355X fp32 vector (the all-fp32 layer runs its GEMMs on the VALU)
METRIC = "tokens/s per K3-shape LatentMoE layer; % MFMA peak (prefill), % HBM BW (decode)"
EXTRA_WORKLOADS = ["k3_decode", "k3_skew", "k3_prefill_mxfp4", "k3_prefill_mx8", "k3_decode_mxfp4",
                   "k3_decode_mx8"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k3_prefill",
                    help="the headline workload (value, roofline, cpu_baseline)")
    ap.add_argument("--extra", default=",".join(EXTRA_WORKLOADS),
                    help="comma-separated workloads timed after the headline one, each reported "
                         "under 'workloads' with its own roofline and CPU baseline ('' = none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the headline oracle baseline sample (0 = skip)")
    ap.add_argument("--cpu-seconds-extra", type=float, default=6.0,
                    help="target CPU time of each extra workload's oracle sample (0 = skip)")
    ap.add_argument("--no-ceilings", dest="ceilings", action="store_false",
                    help="skip the measured MFMA / HBM ceiling probes")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-probe", type=float, default=0.0, metavar="GB",
                    help="instead of the layer: time a plain device-to-device copy of GB "
                         "gigabytes (the reference for HBM rates and PMC byte counters)")
    return ap.parse_args()


def copy_probe(gb: float, steps: int):
    """Plain copy kernel of known size: read gb GB + write gb GB per launch."""
    import torch
    n = int(gb * 1e9) // 16 * 16
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    print(json.dumps({"probe": "device copy", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "ms_per_launch": round(ms, 4),
                      "read_plus_write_GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


GEMM_SRC = os.path.join(ROOT, "sparse_mixture_experts_sigmoid_amd", "csrc", "gemm.hip")
TRAFFIC_MD = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel recorded for `workload`, or
    None if not recorded or recorded on another version of the GEMM source."""
    try:
        text = open(TRAFFIC_MD).read()
        sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    m = re.search(r"traffic-record workload=%s kernel=\S+ gemm_sha=(\w+) bytes=(\d+)" % re.escape(workload),
                  text)
    if not m or m.group(1) != sha:
        return None
    return int(m.group(2))


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, target_s: float):
    """Oracle (route + forward) on growing token samples until ~target_s of work."""
    import numpy as np
    import oracle
    import synth
    w = synth.HostWeights(cfg)
    rng = np.random.default_rng(1234)
    order = rng.permutation(cfg.T)
    done, spent, chunk = 0, 0.0, 1
    while spent < target_s and done < cfg.T:
        toks = np.sort(order[done:done + chunk])
        t0 = time.perf_counter()
        oracle.forward(cfg, w, tokens=toks)          # routes these tokens, then the layer
        spent += time.perf_counter() - t0
        done += len(toks)
        chunk = min(chunk * 2, 64)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(done / spent, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {cfg.T} tokens of {cfg.name} (routing + full layer per token, "
                      f"weights of the touched experts regenerated on the host inside the timing, "
                      f"{spent:.1f} s)"}


PROBE_LIB = os.path.join(ROOT, "sparse_mixture_experts_sigmoid_amd", "libmoe_probe.so")


def measure_ceilings(stream):
    """Measured ceilings of this GPU (libmoe_probe.so): back-to-back bf16
    (32x32x16 and 16x16x32) and MXFP8 x MXFP4 matrix-core instructions with no
    memory traffic, on fixed and on changing operands, and a plain streaming
    read of a 4 GB buffer (16x the 256 MB last-level cache)."""
    import ctypes
    import torch
    L = ctypes.CDLL(PROBE_LIB)
    L.moe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    L.moe_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.moe_probe_mfma_flops.restype = ctypes.c_double
    L.moe_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    sh = stream.cuda_stream

    def timed(fn, reps=5):
        fn()
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    blocks, iters = 256 * 4, 20000                    # 4 waves per SIMD on 256 CUs
    out = torch.empty(blocks * 4, dtype=torch.float32, device="cuda:0")
    res = {}
    for kind, key in ((0, "mfma_bf16_tflops"), (1, "mfma_fp8xfp4_tflops"), (2, "mfma_bf16_changing_data_tflops"),
                      (3, "mfma_fp8xfp4_changing_data_tflops"), (4, "mfma_bf16_16x16x32_tflops"),
                      (5, "mfma_bf16_16x16x32_changing_data_tflops")):
        def launch(kind=kind):
            if L.moe_probe_mfma(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()), sh) != 0:
                raise RuntimeError("moe_probe_mfma failed")
        t = timed(launch)
        res[key] = round(L.moe_probe_mfma_flops(kind, blocks, iters) / t / 1e12, 1)
    # the best of a few launch shapes (blocks per CU x loads in flight per
    # thread, plain or nontemporal loads, spans grid-stride or one contiguous
    # part per block)
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.empty(256 * 16 * 256, dtype=torch.int32, device="cuda:0")
    best = 0.0
    for per_cu in (1, 2, 4, 8):
        for unroll in (4, 8, 16, 0x100 | 8, 0x100 | 16, 0x200 | 8, 0x200 | 16, 0x300 | 8, 0x300 | 16):
            def read(per_cu=per_cu, unroll=unroll):
                if L.moe_probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes, 256 * per_cu, unroll,
                                        ctypes.c_void_p(sink.data_ptr()), sh) != 0:
                    raise RuntimeError("moe_probe_hbm_read failed")
            best = max(best, nbytes / timed(read) / 1e9)
    res["hbm_read_GBps"] = round(best, 1)
    del buf, sink, out
    torch.cuda.empty_cache()
    return res


def workload_string(cfg):
    return (f"{cfg.name}: T={cfg.T} d={cfg.d} d_lat={cfg.d_lat} E={cfg.E} k={cfg.k} F={cfg.F} "
            f"S={cfg.S} Fs={cfg.Fs} act={cfg.act} expert_w={cfg.expert_w} latent_w={cfg.latent_w}"
            + (" expert_act=mxfp8" if cfg.expert_act == "mxfp8" else ""))


def run_workload(name, args, ceilings, cpu_seconds):
    """Time `args.steps` layer calls of workload `name` after `args.warmup`
    untimed ones; returns its record (throughput, roofline of the dominant
    kernel, stage times, CPU oracle baseline)."""
    import torch
    import synth
    import sparse_mixture_experts_sigmoid_amd as moe

    dev = "cuda:0"
    cfg = synth.config(name)
    log(args, f"[bench] {cfg.name}: generating inputs on {dev}")
    # weight-load-time preparation (tiled MXFP4 expert weights where the config
    # asks for them), outside the timed region like the weights themselves
    inp = moe.prepare_weights(cfg, synth.device_inputs(cfg, dev))
    desc = moe.make_desc(cfg)
    act = torch.float32 if cfg.act == "f32" else torch.bfloat16
    y = torch.empty((cfg.T, cfg.d), dtype=act, device=dev)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    counts = torch.empty((cfg.E,), dtype=torch.int32, device=dev)
    ws = moe.workspace(desc, moe.MOE_OP_LAYER, dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_layer_forward(desc, inp, inp["x"], y, idx, gate, counts, ws, stream)

    log(args, f"[bench] {cfg.name}: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: only the dominant stage carries HIP events (each event
    # costs the call a few microseconds)
    moe.moe_trace_enable(args.steps, stages=["expert_gate_up"])
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    timed_stages, ncalls = moe.moe_trace_read()
    # stage breakdown: a few more calls with every stage traced, after the timed region
    nbreak = min(args.steps, 5)
    moe.moe_trace_enable(nbreak)
    for _ in range(nbreak):
        step()
    torch.cuda.synchronize()
    stages, _ = moe.moe_trace_read()
    moe.moe_trace_enable(0)
    stages["expert_gate_up"] = timed_stages["expert_gate_up"]
    log(args, f"[bench] {cfg.name}: {ms:.3f} ms/step; stages " +
        ", ".join(f"{k} {v:.3f}" for k, v in stages.items()))

    cnt = counts.cpu().numpy()
    del inp, y, idx, gate, counts, ws
    torch.cuda.empty_cache()
    touched = int((cnt > 0).sum())
    rows = cfg.T * cfg.k
    wbytes = {"bf16": 2.0, "f32": 4.0, "mxfp4": 0.5 + 1.0 / 32}[cfg.expert_w]
    abytes = 4 if cfg.act == "f32" else 2
    t_gu = stages["expert_gate_up"] * 1e-3
    decode = cfg.T <= 1024
    mx8 = cfg.expert_act == "mxfp8"
    gu_name = ("expert_gate_up (MXFP8 quantise of z + scaled-MFMA grouped GEMM + SiTU-GLU)" if mx8
               else "expert_gate_up (grouped GEMM + SiTU-GLU)")
    if decode:
        # weights of the touched experts + per routed row its z row in and its h
        # row out (bf16, or MXFP8 codes and scales on the scaled-MFMA path)
        zrow = cfg.d_lat * (1 + 1 / 32) if mx8 else cfg.d_lat * abytes
        hrow = cfg.F * (1 + 1 / 32) if mx8 else cfg.F * abytes
        algo = touched * 2 * cfg.F * cfg.d_lat * wbytes + rows * (zrow + hrow)
        achieved = algo / t_gu / 1e9
        meas = ceilings.get("hbm_read_GBps")
        roof = {"bound": "hbm", "kernel": gu_name,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(cfg.name),
                "algorithmic_bytes_per_launch": int(algo), "avg_launch_ms": round(t_gu * 1e3, 4),
                "measured_peak": meas,
                "frac_of_measured": round(achieved / meas, 4) if meas else None}
    else:
        algo = rows * 2 * 2 * cfg.d_lat * cfg.F
        achieved = algo / t_gu / 1e12
        f32 = cfg.act == "f32"
        peak = MFMA_FP8_PEAK_TFLOPS if mx8 else VALU_FP32_PEAK_TFLOPS if f32 else MFMA_BF16_PEAK_TFLOPS
        # the best rate the matrix cores reach alone on this GPU (bf16: either instruction shape)
        meas = (None if f32 else ceilings.get("mfma_fp8xfp4_tflops") if mx8 else
                max((v for v in (ceilings.get("mfma_bf16_tflops"), ceilings.get("mfma_bf16_16x16x32_tflops"))
                     if v), default=None))
        roof = {"bound": "alu" if f32 else "mfma",
                "kernel": gu_name,
                "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(cfg.name),
                "algorithmic_flops_per_launch": int(algo), "avg_launch_ms": round(t_gu * 1e3, 4),
                "measured_peak": meas,
                "frac_of_measured": round(achieved / meas, 4) if meas else None}

    touched_bytes = touched * 3 * cfg.F * cfg.d_lat * wbytes
    layer = {
        "tflops": round(cfg.flops_per_token * cfg.T / (ms * 1e-3) / 1e12, 2),
        "frac_of_mfma_peak": round(cfg.flops_per_token * cfg.T / (ms * 1e-3) / 1e12 /
                                   (MFMA_FP8_PEAK_TFLOPS if mx8 else MFMA_BF16_PEAK_TFLOPS), 4),
        "touched_expert_GBps": round(touched_bytes / (ms * 1e-3) / 1e9, 1),
        "touched_experts": touched,
        "stage_ms": {k: round(v, 4) for k, v in stages.items()},
        "traced_calls": ncalls,
        "stage_ms_source": (f"expert_gate_up: HIP events of the {ncalls} timed calls (their only events); "
                            f"other stages: {nbreak} calls traced stage by stage after the timed region"),
    }
    base = None
    if cpu_seconds > 0:
        log(args, f"[bench] {cfg.name}: cpu baseline (oracle)")
        base = cpu_baseline(cfg, cpu_seconds)
    return {
        "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "dtype": "mxfp8 x mxfp4 experts, bf16 rest" if mx8 else cfg.act,
        "workload": workload_string(cfg), "tokens": cfg.T,
        "roofline": roof, "cpu_baseline": base, "layer": layer,
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the layer's hot path is measured on a single "
                                   "MI355X (the expert-parallel layout across GPUs is a design, not "
                                   "code); use --gpus 1"}))
        return 2

    if args.copy_probe > 0:
        copy_probe(args.copy_probe, args.steps)
        return 0

    import torch
    stream = torch.cuda.current_stream()
    ceilings = measure_ceilings(stream) if args.ceilings else {}
    if ceilings:
        log(args, f"[bench] measured ceilings {ceilings}")

    head = run_workload(args.workload, args, ceilings, args.cpu_seconds)
    extras = {}
    for name in [n for n in args.extra.split(",") if n and n != args.workload]:
        extras[name] = run_workload(name, args, ceilings, args.cpu_seconds_extra)

    out = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic: seeded counter-based N(0,1) activations and N(0,1/fan_in) "
                "random-init weights of the K3 layer shape (no checkpoint)",
        "config": {"workload": head["workload"], "tokens": head["tokens"],
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "layer": head["layer"],
        "ceilings": ceilings or None,
        "workloads": extras,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
