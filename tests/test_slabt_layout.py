"""CPU-only: the index arithmetic of the GEMM core's transposed slab operand.

dZ reads each chunk's state W_i and state gradient Gbar (sb<256>(d x f)
matrices) as its B operand with K over their rows: direct-to-LDS loads copy
1 KB blocks of the sb image into a permuted LDS image, and LDS transpose
reads (ds_read_b64_tr_b16) assemble the MFMA fragments. The layout functions
(slabt_* in ttt_launch.h) are host+device code; slabt_layout_check.cpp
compiles them for the host, emulates the loads and the transpose read's lane
semantics on a matrix whose elements hold their own coordinates, and checks
every fragment element, every piece's bounds and the reads' bank use.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "test_layer_gate_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def test_transposed_slab_layout(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("g++ or the HIP headers are not installed")
    exe = tmp_path / "slabt_layout_check"
    res = subprocess.run([gxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
                          "-I", CSRC, os.path.join(ROOT, "tests", "slabt_layout_check.cpp"),
                          "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
