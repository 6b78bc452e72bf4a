"""Build libttt_layer.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m test_layer_gate_amd.build

Every call recompiles. The result sits next to this file so that it travels
with the source tree; nothing is installed elsewhere.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libttt_layer.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["ttt_kernels.hip", "ttt_decode.hip", "ttt_backward.hip", "ttt_noalloc.hip",
           "ttt_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libttt_layer)")


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed-fp32 VALU forms stay off: hipcc would otherwise emit them
           # from ordinary float code.
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", INCLUDE, "-I", CSRC, "-o", tmp]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
