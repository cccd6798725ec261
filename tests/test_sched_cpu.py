"""The grouped GEMM's schedule and operand addresses, checked on the host.

tests/sched_check.cpp includes the kernels' own header (gemm_sched.h) and checks, with no GPU:
every LDS-DMA source stays inside its operand row or tiled block for every K in [8, 65536];
every output tile is computed exactly once by the single and the split launches; the split
tail's reducer sums exactly the K pieces the GEMM launch wrote for the same tiles.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_19_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_schedule_and_addresses(tmp_path):
    exe = tmp_path / "sched_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(ROOT, "tests", "sched_check.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok "), res.stdout
