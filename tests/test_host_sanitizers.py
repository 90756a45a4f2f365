"""The C-ABI library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: every argument check of include/dit_attn.h runs
from a C++ driver (tests/host_sanitizer_driver.cpp) linked against a build
of the library whose host code is instrumented (the device code is built as
usual and never launched: every case fails validation before any HIP call,
so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_sequence_attention_amd", "csrc")
SOURCES = ["api.hip", "attn_fwd.hip", "elementwise.hip", "fixed_m.hip"]


def test_argument_checks_are_clean_under_host_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "host_sanitizer_driver")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES],
           os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if res.returncode != 0 and "asan" in (res.stderr or "").lower() and "cannot find" in (res.stderr or "").lower():
        pytest.skip("sanitizer runtime not installed")
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0 and "ALL OK" in run.stdout, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
