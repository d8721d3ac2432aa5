"""Sanitizer builds of the host-side code, run without a GPU:
- the CPU oracle (oracle/oracle.c) and the host twin of the input generator
  (synth/csrc/synth_host.c), built with AddressSanitizer and
  UndefinedBehaviorSanitizer by gcc and driven on small shapes and edge values
  by tests/sanitize/driver.c;
- the library's host code (csrc/abi.hip) built with the same sanitizers on
  its host side, under every host-side ABI test.
Any out-of-bounds access, overflow or other undefined operation fails them."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitized")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "driver.c"),
            os.path.join(ROOT, "oracle", "oracle.c"),
            os.path.join(ROOT, "synth", "csrc", "synth_host.c")]
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-o", exe, *srcs, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


ASAN_RT_GLOB = "/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_abi_host_validation_under_asan_ubsan(tmp_path):
    """The library's host code (csrc/abi.hip: descriptor and argument
    validation, workspace planning, the layouts' size helpers) built with
    AddressSanitizer and UndefinedBehaviorSanitizer on the host side only
    (the kernels are the in-tree objects), then every host-side ABI test
    (tests/test_abi_host.py) run against it in a child process with the
    sanitizer runtime preloaded. No GPU call is made."""
    import glob
    import sys
    from sparse_mixture_experts_sigmoid_amd import build as B
    others = [os.path.join(B.BUILD, s.replace(".hip", ".o")) for s in B.SOURCES if s != "abi.hip"]
    rt = sorted(glob.glob(ASAN_RT_GLOB))
    if not all(os.path.exists(o) for o in others) or not rt:
        pytest.skip("needs the in-tree objects (build()) and clang's ASan runtime")
    obj, lib = str(tmp_path / "abi_asan.o"), str(tmp_path / "libmoe_asan.so")
    flags = [f for f in B.FLAGS if f != "-O3"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    subprocess.run([B.HIPCC, *flags, "-O1", "-g", "-fno-omit-frame-pointer", *san,
                    "-Xarch_host", "-fno-sanitize-recover=all",
                    "-c", os.path.join(B.CSRC, "abi.hip"), "-o", obj], check=True, capture_output=True)
    subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", *san,
                    "-o", lib, obj, *others], check=True, capture_output=True)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "abi.o is not instrumented"
    # reports go to files: the child's pytest would capture them on fd 2 and
    # lose them when the sanitizer ends the process
    logs = tmp_path / "san"
    env = dict(os.environ, LD_PRELOAD=rt[-1], MOE_LIB_PATH=lib,
               ASAN_OPTIONS=f"detect_leaks=0:verify_asan_link_order=0:log_path={logs}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={logs}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    reports = "".join(open(f).read() for f in glob.glob(f"{logs}*"))
    assert reports == "", reports[-4000:]
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
