"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer: the
library's sources and a driver (tests/sanitize/abi_refusals.cpp) that calls every entry point
with arguments it must refuse, and the workspace-size functions at and past their limits, are
built with the sanitizers on the host code (the device code is compiled as usual and never
runs) and executed; any sanitizer report or unexpected status fails the test."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


def test_abi_refusals_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_refusals")
    srcs = sorted(glob.glob(os.path.join(ROOT, "denoise_step_sampler_amd", "csrc", "*.hip")))
    cmd = ["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "denoise_step_sampler_amd", "csrc"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-static-libsan",
           *srcs, os.path.join(ROOT, "tests", "sanitize", "abi_refusals.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "0 failed expectations" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
