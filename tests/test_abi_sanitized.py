"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/plan_errors.cpp drives every validation error of vsa_plan,
valid plans of each mask policy (info, workspace regions), and the argument
checks of the execution and getter entry points that end before any device
access.  It is linked with csrc/api.cpp (host code instrumented) and host-only
stand-ins for the kernel launchers, so it runs without a GPU.  Needs hipcc.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = [os.path.join(ROOT, "block_sparse_attention_tile_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launcher_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "plan_errors.cpp")]
# the sanitizers instrument host code only (each flag after -Xarch_host)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_plan_and_argument_errors_under_asan_ubsan(tmp_path):
    objs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
               "-Xarch_host", "-fno-omit-frame-pointer"] + SAN + ["-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(tmp_path / "plan_errors")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950"] + SAN + objs + ["-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
