"""CPU-only: the gfx950 assembly of the kernels, compiled here from source.

The direct-to-LDS loads set M0 (the LDS address) in inline asm, and the
compiler does not honour M0 in an asm clobber list. That is safe only while
no compiler-generated instruction uses M0 between such a write and its load.
This test compiles the kernel sources for gfx950 and checks that every
instruction that names M0, or reads it implicitly, is part of the pattern
the inline asm writes: `s_mov_b32 m0, sN`, `s_nop 0`, then the
`buffer_load_dwordx4 ... offen lds` that consumes it.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "test_layer_gate_amd", "csrc")
SOURCES = ["ttt_kernels.hip", "ttt_decode.hip", "ttt_backward.hip"]

# instructions that read M0 without naming it
IMPLICIT_M0 = re.compile(r"^(s_sendmsg|s_sendmsghalt|s_movrel|v_movrel|v_interp|ds_gws|"
                         r"ds_ordered|global_load_lds|buffer_load_\w+\s.*\blds$|"
                         r"buffer_store_lds|s_ttracedata)")
M0_WRITE = re.compile(r"^s_mov_b32 m0, s\d+$")
DMA_LOAD = re.compile(r"^buffer_load_dwordx4 v\d+, s\[\d+:\d+\], s\d+ offen lds$")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.parametrize("src", SOURCES)
def test_m0_only_feeds_the_direct_to_lds_loads(tmp_path, src):
    cc = hipcc()
    if cc is None:
        pytest.skip("hipcc is not installed")
    out = tmp_path / (src + ".s")
    res = subprocess.run([cc, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only",
                          "-S", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                          os.path.join(CSRC, src), "-o", str(out)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    ins = [ln.split(";")[0].strip() for ln in out.read_text().split("\n")]
    ins = [i for i in ins if i and not i.startswith(".") and not i.endswith(":")]
    n_loads = 0
    for k, i in enumerate(ins):
        names_m0 = re.search(r"\bm0\b", i) is not None
        if not names_m0 and not IMPLICIT_M0.match(i):
            continue
        if M0_WRITE.match(i):
            assert k + 2 < len(ins) and ins[k + 1] == "s_nop 0" and DMA_LOAD.match(ins[k + 2]), \
                f"M0 write not followed by its load: {ins[k:k + 3]}"
            continue
        if DMA_LOAD.match(i):
            assert k >= 2 and M0_WRITE.match(ins[k - 2]) and ins[k - 1] == "s_nop 0", \
                f"direct-to-LDS load without its own M0 write: {ins[k - 2:k + 1]}"
            n_loads += 1
            continue
        pytest.fail(f"compiler-generated M0 use: {i!r} (instruction {k})")
    if src in ("ttt_kernels.hip", "ttt_backward.hip"):
        assert n_loads > 100, "the GEMM core's direct-to-LDS loads are missing"
