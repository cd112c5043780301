"""Argument validation and workspace layout (csrc/kd_plan.cpp) under the host
compiler's AddressSanitizer and UndefinedBehaviorSanitizer.

tests/plan_check.cpp walks a grid of valid, edge and invalid shapes for every
pass, up to and past the 32-bit limits the kernels state, and checks that each
accepted plan gives every region the kernels index a 256-byte aligned,
in-bounds, non-overlapping place in the workspace; a signed overflow in the
size arithmetic aborts the run. Host code only: nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_kl_loss_chunk_amd", "csrc")


def _cxx():
    return shutil.which("g++") or shutil.which("c++")


@pytest.mark.skipif(_cxx() is None, reason="no host C++ compiler")
@pytest.mark.parametrize("sanitize", ["address,undefined", None])
def test_plan_layout_under_sanitizers(tmp_path, sanitize):
    exe = tmp_path / "plan_check"
    cmd = [_cxx(), "-std=c++17", "-O1", "-g", "-Wall", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "plan_check.cpp"), os.path.join(CSRC, "kd_plan.cpp"),
           "-o", str(exe)]
    if sanitize:
        cmd[1:1] = [f"-fsanitize={sanitize}", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if sanitize and res.returncode != 0 and "sanitizer" in (res.stderr or "").lower():
        pytest.skip(f"sanitizer runtime not available: {res.stderr[-300:]}")
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout, run.stdout
    valid = int(run.stdout.split("plans: ")[1].split()[0])
    assert valid > 1000, run.stdout
