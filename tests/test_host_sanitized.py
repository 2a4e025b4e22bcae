"""The plan code built with AddressSanitizer and UndefinedBehaviorSanitizer
(host compiler only, no device code) and driven over host-only plans from a
1x1 grid to 8K, ragged grids, both LR modes and radii up to 4, every host
export, descriptor validation, and the hand-out order of the work-queue
cursor slots (tests/host/plan_driver.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_transformer_sparse_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "plan_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, "-I/opt/rocm/include", os.path.join(ROOT, "tests", "host", "plan_driver.cpp"),
           os.path.join(CSRC, "plan.cpp"), "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-2000:], r.stderr[-4000:])
