"""Invariants of the launch planner and its plan cache (host only, no GPU).

Builds tests/plan_check.cpp against the library's planner source with g++ and the
address and undefined-behaviour sanitizers, and runs it: every row's keys covered
exactly once by the work list, split key ranges merged exactly once over written
partial slots, slots disjoint, split pieces within the per-wave id budget, the
fused append's copying workgroups counted, each chunk group on a contiguous run
of die lanes. Builds tests/plan_cache_check.cpp the same way, and
once more under the thread sanitizer for its many-thread lookups: cached records
equal fresh plans, keys tell every shape apart, least-recently-used eviction and
the bounds hold.
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


def _build(tmp_path, name, main_src, sanitizers):
    exe = tmp_path / name
    csrc = os.path.join(ROOT, "chunked_prefill_attention_extend_amd", "csrc")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), f"-fsanitize={sanitizers}", "-fno-sanitize-recover=all",
           os.path.join(HERE, main_src), os.path.join(csrc, "plan.cpp"), os.path.join(csrc, "plan_cache.cpp"),
           "-o", str(exe), "-lpthread"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    return exe


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_cache_records_keys_and_bounds(tmp_path):
    exe = _build(tmp_path, "plan_cache_check", "plan_cache_check.cpp", "address,undefined")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, (run.stdout[-3000:] + run.stderr[-3000:])
    assert "0 failures" in run.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_cache_threads_race_free(tmp_path):
    exe = _build(tmp_path, "plan_cache_check_tsan", "plan_cache_check.cpp", "thread")
    run = subprocess.run([str(exe), "threads"], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, (run.stdout[-3000:] + run.stderr[-3000:])
    assert "0 failures" in run.stdout and "ThreadSanitizer" not in run.stderr
