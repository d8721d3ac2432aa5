"""Build the generator twins: libsynth_host.so (gcc) and libsynth_dev.so (hipcc, gfx950)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    subprocess.run(cmd, check=True)


def build_host():
    _run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-o", os.path.join(HERE, "libsynth_host.so"),
          os.path.join(HERE, "csrc", "synth_host.c"), "-lm"])


def build_device():
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
          "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-o", os.path.join(HERE, "libsynth_dev.so"),
          os.path.join(HERE, "csrc", "synth_dev.hip")])


def build():
    build_host()
    build_device()


if __name__ == "__main__":
    build()
