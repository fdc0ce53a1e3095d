"""The library's host-only planning code (csrc/host_plan.cpp: argument validation, the sampling step's
row plan, the attention work split and the workspace layout) built on its own with g++ under the
address and undefined-behaviour sanitizers, and driven by tests/host_plan_check.cpp: validation fuzz,
and for every accepted step and forward over a grid of shapes, batches and guidance settings, a check
that the workspace holds what that call's kernels write (no GPU, no HIP)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_transformer_text_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_plan_under_asan_ubsan(tmp_path):
    exe = tmp_path / "host_plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_plan_check.cpp"), os.path.join(CSRC, "host_plan.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) > 100000
