"""Launch-plan cache policy on the host (no GPU): least-recently-used
eviction, and pinning of plans that a captured HIP graph refers to."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "newton_schulz_flat_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_cache_policy(tmp_path):
    exe = tmp_path / "plan_cache_check"
    src = os.path.join(ROOT, "tests", "plan_cache_check.cpp")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror",
                    "-fsanitize=address,undefined", f"-I{CSRC}", src, "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip() == "ok"
