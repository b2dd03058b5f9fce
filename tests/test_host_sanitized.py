"""The library's host planning code (plan.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/host_plan_check.cpp drives it over random
and edge-case arguments (schedule bounds, no conflicting transfers within a
step, closed-form byte counts equal the schedules' counts, chunk tiling,
argument validation).  Built with the host C++ compiler; no GPU code."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_allreduce_algorithms_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_plan_code_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "host_plan_check")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "host_plan_check.cpp"),
         "-o", exe],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    # the process environment is kept as it is; ASan is told not to insist on
    # being first in the library load order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout[-4000:] + run.stderr[-4000:])
    assert run.stdout.strip().splitlines()[-1].startswith("OK")
