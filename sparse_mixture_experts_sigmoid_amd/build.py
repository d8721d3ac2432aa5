"""Build libmoe.so (the C-ABI library of the gfx950 kernels) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build", "moe")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["abi.hip", "router.hip", "permute.hip", "gemm.hip", "gemm_f32.hip", "combine.hip",
           "qb.hip", "mx8.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
         "-Wall", "-Wno-unused-function",
         # packed fp32 vector ops stay off in every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    r = subprocess.run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


# ceiling probes for the benchmark (not part of the layer): libmoe_probe.so
PROBE_SOURCES = ["probe.hip"]
PROBE_OUT = os.path.join(HERE, "libmoe_probe.so")


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    n = len(SOURCES)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", OUT, *objs[:n]],
                   check=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", PROBE_OUT, *objs[n:]],
                   check=True)
    return OUT


if __name__ == "__main__":
    print(build())
