"""The host plan (linear_cross_entropy_lm_amd/csrc/flce_plan.h: size limits, workspace
layouts, chunk choice, 32-bit buffer-descriptor bounds) compiled on the CPU with g++ under
AddressSanitizer and UBSan, and its checks run: the closed-form descriptor bounds against a
brute-force enumeration of the kernels' load offsets, a sweep of sizes x dtypes x
workspaces in which every chosen plan keeps its operands within the descriptor limit and
its writes within their workspace regions, and the configurations that overflowed before
the caps existed.  No GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "plan_check.cpp")
INC = os.path.join(ROOT, "linear_cross_entropy_lm_amd", "csrc")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror", *SANITIZE, "-I", INC, SRC, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stdout + build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                              "UBSAN_OPTIONS": "print_stacktrace=1"})
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all plan checks passed" in run.stdout
