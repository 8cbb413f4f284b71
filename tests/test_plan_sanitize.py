"""Host-only sanitizer build of the launch planner (CPU).

w4a16_weight_only_amd/csrc/awq_plan.cpp (argument checks, family choice, launch shapes,
workspace sizes) is compiled with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
together with tests/plan_check.cpp, which sweeps about 2.4 million shapes (edge sizes from
0 and the format's limits to INT64_MIN / INT64_MAX, random in-range shapes, routed-expert
and RTN-writer plans, pack validation) and checks each plan against the kernels'
contracts: launch limits, coverage of every tile and k-step, split counts, group spans,
32-bit offsets and workspace sizes.  Any sanitizer report aborts the run.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def plan_check(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan_san") / "plan_check")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-static-libasan", "-static-libubsan", "-Wall", "-Wextra", "-Werror",
           os.path.join(ROOT, "tests", "plan_check.cpp"),
           os.path.join(ROOT, "w4a16_weight_only_amd", "csrc", "awq_plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return exe


def test_planner_sweep_under_asan_ubsan(plan_check):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([plan_check], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout, r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    n = int(r.stdout.split("plans checked:")[1].split()[0])
    assert n > 2_000_000
