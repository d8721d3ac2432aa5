"""The CPU oracle (oracle/oracle.c) and the host twin of the input generator
(synth/csrc/synth_host.c) built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only) and run on small shapes and
edge values by tests/sanitize/driver.c: any out-of-bounds access, overflow or
other undefined operation in them fails this test."""
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
