"""Invariants of the launch planner on random launches (host only, no GPU).

Builds tests/plan_check.cpp against the library's planner source with g++ and the
address and undefined-behaviour sanitizers, and runs it: every row's keys covered
exactly once by the work list, split key ranges merged exactly once over written
partial slots, slots disjoint, split pieces within the per-wave id budget, fused
append items first and covering every new token once, each chunk group on a
contiguous run of die lanes.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_invariants(tmp_path):
    exe = tmp_path / "plan_check"
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(HERE, "plan_check.cpp"),
           os.path.join(ROOT, "chunked_prefill_attention_extend_amd", "csrc", "plan.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe), "120"], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, (run.stdout[-3000:] + run.stderr[-3000:])
    assert "0 failures" in run.stdout
