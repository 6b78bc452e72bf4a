"""CPU-only: the C-ABI library loads, exports every function include/ttt.h
declares, and rejects bad arguments on the host before launching anything.

No call here reaches a kernel launch: every call fails argument checking,
which runs before any HIP call. Pointers are fake, aligned addresses that the
library never dereferences on an error path.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")

from test_layer_gate_amd import _binding as bnd  # noqa: E402

OK, INVALID, UNSUPPORTED, WORKSPACE, ALIAS = 0, -1, -2, -3, -4


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    names = set(re.findall(r"\b(ttt_[a-z_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bnd.LIB_PATH):
        pytest.fail("libttt_layer.so is not built (run __graft_entry__.build())")
    return bnd.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in ttt.h but not exported"


# The boundary the survey sketched (its names) and the exported function
# that serves each; where the name differs, the design doc's boundary table gives
# the reason (the survey's debug calls took no workspace, and its size call
# had no way to report an invalid descriptor).
SURVEY_BOUNDARY = {
    "ttt_workspace_size": "ttt_workspace_size",
    "ttt_layer_forward": "ttt_layer_forward",
    "ttt_status_string": "ttt_status_string",
    "ttt_last_error_message": "ttt_last_error_message",
    "ttt_debug_gate_up": "ttt_gated_activation",
    "ttt_debug_target": "ttt_lm_target",
}


def header_constants():
    src = open(HEADER).read()
    return {k: v for k, v in re.findall(r"\b(TTT_[A-Z0-9_]+)\s*=\s*([-0-9a-fx<u ]+?)\s*[,}\n/]",
                                          src)}


def test_survey_boundary_is_served(L):
    declared = set(declared_functions())
    for survey_name, ours in SURVEY_BOUNDARY.items():
        assert ours in declared, f"{survey_name}: {ours} is not declared in ttt.h"
        assert hasattr(L, ours), f"{survey_name}: {ours} is not exported"
    c = header_constants()
    want = {"TTT_OK": "0", "TTT_ERR_INVALID_ARG": "-1", "TTT_ERR_UNSUPPORTED": "-2",
            "TTT_ERR_WORKSPACE": "-3", "TTT_ERR_ALIAS": "-4", "TTT_ERR_HIP": "-5",
            "TTT_BF16": "0", "TTT_F32": "1", "TTT_FLAG_PAD_CHUNK": "1u << 0",
            "TTT_FLAG_SCHED_RUNNING": "1u << 1", "TTT_FLAG_SCHED_PREFIX": "1u << 2"}
    for k, v in want.items():
        assert c.get(k, "").strip() == v, (k, c.get(k))


def test_last_error_message_is_last_error(L):
    L.ttt_last_error_message.restype = ctypes.c_char_p
    st, _ = ws_size(L, qwen_desc(batch=0), 1024)
    assert st == INVALID
    assert L.ttt_last_error_message() == L.ttt_last_error() == b"batch must be >= 1"


def test_status_strings(L):
    for code, name in [(0, "TTT_OK"), (-1, "TTT_ERR_INVALID_ARG"), (-2, "TTT_ERR_UNSUPPORTED"),
                       (-3, "TTT_ERR_WORKSPACE"), (-4, "TTT_ERR_ALIAS"), (-5, "TTT_ERR_HIP")]:
        assert L.ttt_status_string(code).decode() == name


def qwen_desc(**kw):
    a = dict(batch=1, seq_len=65536, d_model=2560, d_ff=9728, conv_k=4)
    a.update(kw)
    return bnd.make_desc(**a)


def ws_size(L, desc, chunk):
    n = ctypes.c_size_t(0)
    st = L.ttt_workspace_size(ctypes.byref(desc), chunk, ctypes.byref(n))
    return st, n.value


def test_workspace_size_matches_layout(L):
    st, n = ws_size(L, qwen_desc(), 1024)
    assert st == OK
    B, T, d, f, k = 1, 65536, 2560, 9728, 64

    def pad(x):  # rows padded to an odd number of 128-byte lines
        return x + 64 if (x // 64) % 2 == 0 else x
    ld_y, ld_f = pad(d), pad(f)
    def sb(rows, K, SR):  # slab-blocked: whole SR-row slabs
        return -(-rows // SR) * SR * K
    # Y, W_target^T, Z, Z^T and V^T, snapshots, packed W_g and W_u (whole
    # 128-row slabs)
    expect = (B * T * ld_y * 2 + d * ld_y * 2 + B * T * ld_f * 2 + B * sb(f, T, 256) * 2
              + B * sb(d, T, 256) * 2 + B * k * sb(d, f, 256) * 2
              + 2 * (-(-f // 128) * 128) * d * 2
              + 4 * 256 * 4)     # the fp16 operand-range buffer
    assert expect <= n <= expect + 16 * 256
    st, n_run = ws_size(L, qwen_desc(flags=bnd.FLAG_SCHED_RUNNING), 1024)
    assert st == OK and n_run < n      # running schedule keeps one bf16 copy


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, INVALID), ("seq_len", 0, INVALID), ("d_model", 0, INVALID),
    ("d_ff", -64, INVALID), ("conv_k", 0, INVALID), ("act_dtype", 7, INVALID),
    ("weight_dtype", -1, INVALID), ("flags", 1 << 9, INVALID),
    ("flags", bnd.FLAG_SCHED_RUNNING | bnd.FLAG_SCHED_PREFIX, INVALID),
    ("w0_batch_stride", -1, INVALID), ("w0_batch_stride", 100, INVALID),
    ("d_model", 2500, UNSUPPORTED), ("d_ff", 9700, UNSUPPORTED), ("conv_k", 65, UNSUPPORTED),
])
def test_bad_descriptor(L, field, value, code):
    desc = qwen_desc()
    setattr(desc, field, value)
    st, _ = ws_size(L, desc, 1024)
    assert st == code, (field, value, st, L.ttt_last_error())
    assert L.ttt_last_error().decode()


@pytest.mark.parametrize("chunk,code", [(0, INVALID), (-64, INVALID), (100, UNSUPPORTED),
                                        (64, OK), (1024, OK)])
def test_chunk_validation(L, chunk, code):
    st, _ = ws_size(L, qwen_desc(), chunk)
    assert st == code


class FakeBuffers:
    """Distinct, 256-byte aligned fake device addresses, far apart."""

    def __init__(self):
        self.base = 1 << 40
        self.step = 1 << 36

    def __getitem__(self, i):
        return ctypes.c_void_p(self.base + i * self.step)


def forward(L, desc, ptrs, eta=1e-3, chunk=1024, ws_bytes=1 << 62):
    return L.ttt_layer_forward(ctypes.byref(desc), *ptrs[:7], ctypes.c_float(eta), chunk,
                               ptrs[7], ptrs[8], ptrs[9], ctypes.c_size_t(ws_bytes), None)


def good_ptrs():
    fb = FakeBuffers()
    return [fb[i] for i in range(10)]


def test_forward_rejects_nonfinite_eta(L):
    assert forward(L, qwen_desc(), good_ptrs(), eta=float("nan")) == INVALID
    assert forward(L, qwen_desc(), good_ptrs(), eta=float("inf")) == INVALID


@pytest.mark.parametrize("idx", range(10))
def test_forward_rejects_null(L, idx):
    p = good_ptrs()
    p[idx] = ctypes.c_void_p(0)
    assert forward(L, qwen_desc(), p) == INVALID
    assert "NULL" in L.ttt_last_error().decode()


@pytest.mark.parametrize("idx", range(10))
def test_forward_rejects_misaligned(L, idx):
    p = good_ptrs()
    p[idx] = ctypes.c_void_p(p[idx].value + 8)
    assert forward(L, qwen_desc(), p) == INVALID
    assert "aligned" in L.ttt_last_error().decode()


def test_forward_rejects_small_workspace(L):
    _, need = ws_size(L, qwen_desc(), 1024)
    assert forward(L, qwen_desc(), good_ptrs(), ws_bytes=need - 1) == WORKSPACE


@pytest.mark.parametrize("out_idx,in_idx", [(7, 0), (7, 1), (8, 4), (8, 2), (9, 6), (7, 8),
                                            (9, 7)])
def test_forward_rejects_aliasing(L, out_idx, in_idx):
    p = good_ptrs()
    p[out_idx] = ctypes.c_void_p(p[in_idx].value + 4096)
    st = forward(L, qwen_desc(), p)
    assert st == ALIAS, L.ttt_last_error()


def test_step_entry_points_validate(L):
    desc = qwen_desc()
    fb = FakeBuffers()
    st = L.ttt_gated_activation(ctypes.byref(desc), fb[0], fb[1], ctypes.c_void_p(0), fb[3],
                                fb[4], ctypes.c_size_t(1 << 62), None)
    assert st == INVALID
    st = L.ttt_lm_target(ctypes.byref(desc), fb[0], fb[1], fb[2], 100, fb[3], fb[4],
                         ctypes.c_size_t(1 << 62), None)
    assert st == UNSUPPORTED
    st = L.ttt_lm_target(ctypes.byref(desc), fb[0], fb[1], fb[2], 1024, fb[3], fb[4],
                         ctypes.c_size_t(16), None)
    assert st == WORKSPACE


def test_binding_without_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bnd, "_lib", None)
    monkeypatch.setattr(bnd, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        bnd.lib()


# ---- packed documents --------------------------------------------------------

def packed_ws(L, desc, chunk, starts):
    arr = (ctypes.c_int32 * max(len(starts), 1))(*starts) if starts is not None else None
    n = ctypes.c_size_t(0)
    st = L.ttt_packed_workspace_size(ctypes.byref(desc), chunk, arr,
                                     len(starts) if starts is not None else 1, ctypes.byref(n))
    return st, n.value


def test_packed_workspace_size(L):
    desc = qwen_desc()
    starts = [0, 1024 * 10, 1024 * 10 + 64, 40000 - 40000 % 64]
    st, n = packed_ws(L, desc, 1024, starts)
    assert st == OK, L.ttt_last_error()
    _, plain = ws_size(L, desc, 1024)
    T, d, f = 65536, 2560, 9728
    ends = starts[1:] + [T]
    k = sum(-(-(e - a) // 1024) for a, e in zip(starts, ends))
    snap = -(-d // 256) * 256 * f * 2
    chunks = [(t, min(e, t + 1024)) for a, e in zip(starts, ends) for t in range(a, e, 1024)]
    n_tiles = sum(-(-(t1 - t0) // 256) for t0, t1 in chunks)
    assert len(chunks) == k
    # more chunks, plus the block table, the apply's tile list and the chunk spans
    extra = (k - 64) * snap + T // 64 * 16 + n_tiles * 16 + k * 8
    assert plain + extra <= n <= plain + extra + 4 * 256


@pytest.mark.parametrize("starts,code", [
    ([0], OK), ([0, 64, 128], OK), ([64], INVALID), ([0, 128, 128], INVALID),
    ([0, 256, 128], INVALID), ([0, 65536], INVALID), ([0, 100], UNSUPPORTED),
    ([], INVALID), (None, INVALID)])
def test_packed_document_validation(L, starts, code):
    st, _ = packed_ws(L, qwen_desc(), 1024, starts)
    assert st == code, (starts, st, L.ttt_last_error())


def test_packed_needs_batch_one(L):
    st, _ = packed_ws(L, qwen_desc(batch=2), 1024, [0, 64])
    assert st == UNSUPPORTED


def test_packed_forward_validates_before_launch(L):
    desc = qwen_desc()
    p = good_ptrs()
    starts = (ctypes.c_int32 * 2)(0, 100)
    st = L.ttt_layer_forward_packed(ctypes.byref(desc), *p[:7], ctypes.c_float(1e-3), 1024,
                                    starts, 2, p[7], p[8], p[9], ctypes.c_size_t(1 << 62), None)
    assert st == UNSUPPORTED
    starts = (ctypes.c_int32 * 2)(0, 128)
    _, need = packed_ws(L, desc, 1024, [0, 128])
    st = L.ttt_layer_forward_packed(ctypes.byref(desc), *p[:7], ctypes.c_float(1e-3), 1024,
                                    starts, 2, p[7], p[8], p[9], ctypes.c_size_t(need - 1), None)
    assert st == WORKSPACE


# ---- update-norm clipping ----------------------------------------------------

def clipped_ws(L, desc, chunk, clip):
    n = ctypes.c_size_t(0)
    st = L.ttt_clipped_workspace_size(ctypes.byref(desc), chunk, ctypes.c_float(clip),
                                      ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("clip,code", [(1.0, OK), (1e-6, OK), (0.0, INVALID), (-1.0, INVALID),
                                       (float("inf"), INVALID), (float("nan"), INVALID)])
def test_clip_validation(L, clip, code):
    st, _ = clipped_ws(L, qwen_desc(), 1024, clip)
    assert st == code, (clip, st)


def test_clipped_workspace_size(L):
    st, n = clipped_ws(L, qwen_desc(), 1024, 1.0)
    assert st == OK
    _, plain = ws_size(L, qwen_desc(), 1024)
    T, d, k = 65536, 2560, 64
    ld_y = d + 64 if (d // 64) % 2 == 0 else d
    pairs = 4 * 5 // 2                              # 256-token blocks of a 1024-token chunk
    # token-major V, the V Gram tiles, Gram partials (two parts of d_ff), scales
    extra = T * ld_y * 2 + k * pairs * 256 * 256 * 4 + k * pairs * 2 * 4 + k * 4
    assert plain + extra <= n <= plain + extra + 5 * 256


def test_clipped_forward_validates_before_launch(L):
    p = good_ptrs()
    st = L.ttt_layer_forward_clipped(ctypes.byref(qwen_desc()), *p[:7], ctypes.c_float(1e-3),
                                     1024, ctypes.c_float(0.0), p[7], p[8], p[9],
                                     ctypes.c_size_t(1 << 62), None)
    assert st == INVALID
    _, need = clipped_ws(L, qwen_desc(), 1024, 1.0)
    st = L.ttt_layer_forward_clipped(ctypes.byref(qwen_desc()), *p[:7], ctypes.c_float(1e-3),
                                     1024, ctypes.c_float(1.0), p[7], p[8], p[9],
                                     ctypes.c_size_t(need - 1), None)
    assert st == WORKSPACE


# ---- packed documents with clipping -------------------------------------------

def packed_clipped_ws(L, desc, chunk, starts, clip):
    arr = (ctypes.c_int32 * len(starts))(*starts)
    n = ctypes.c_size_t(0)
    st = L.ttt_packed_clipped_workspace_size(ctypes.byref(desc), chunk, arr, len(starts),
                                             ctypes.c_float(clip), ctypes.byref(n))
    return st, n.value


def test_packed_clipped_workspace_size(L):
    """The packed layout plus the clipped path's buffers, sized by the packed
    chunk count (chunks restart at every document)."""
    desc = qwen_desc()
    starts = [0, 1024 * 10, 1024 * 10 + 64, 40000 - 40000 % 64]
    st, n = packed_clipped_ws(L, desc, 1024, starts, 1.0)
    assert st == OK, L.ttt_last_error()
    _, packed = packed_ws(L, desc, 1024, starts)
    T, d = 65536, 2560
    ends = starts[1:] + [T]
    k = sum(-(-(e - a) // 1024) for a, e in zip(starts, ends))
    ld_y = d + 64 if (d // 64) % 2 == 0 else d
    pairs = 4 * 5 // 2
    extra = T * ld_y * 2 + k * pairs * 256 * 256 * 4 + k * pairs * 2 * 4 + k * 4
    assert packed + extra <= n <= packed + extra + 5 * 256


@pytest.mark.parametrize("starts,clip,code", [
    ([0, 128], 1.0, OK), ([0, 128], 0.0, INVALID), ([0, 128], float("nan"), INVALID),
    ([0, 100], 1.0, UNSUPPORTED), ([64], 1.0, INVALID)])
def test_packed_clipped_validation(L, starts, clip, code):
    st, _ = packed_clipped_ws(L, qwen_desc(), 1024, starts, clip)
    assert st == code, (starts, clip, st, L.ttt_last_error())


def test_packed_clipped_forward_validates_before_launch(L):
    desc = qwen_desc()
    p = good_ptrs()
    starts = (ctypes.c_int32 * 2)(0, 128)
    st = L.ttt_layer_forward_packed_clipped(ctypes.byref(desc), *p[:7], ctypes.c_float(1e-3),
                                            1024, starts, 2, ctypes.c_float(-1.0), p[7], p[8],
                                            p[9], ctypes.c_size_t(1 << 62), None)
    assert st == INVALID
    _, need = packed_clipped_ws(L, desc, 1024, [0, 128], 1.0)
    st = L.ttt_layer_forward_packed_clipped(ctypes.byref(desc), *p[:7], ctypes.c_float(1e-3),
                                            1024, starts, 2, ctypes.c_float(1.0), p[7], p[8],
                                            p[9], ctypes.c_size_t(need - 1), None)
    assert st == WORKSPACE


# ---- continuation ------------------------------------------------------------

def continue_ws(L, desc, chunk):
    n = ctypes.c_size_t(0)
    st = L.ttt_continue_workspace_size(ctypes.byref(desc), chunk, ctypes.byref(n))
    return st, n.value


def test_continue_workspace_size(L):
    st, n = continue_ws(L, qwen_desc(), 1024)
    assert st == OK
    _, plain = ws_size(L, qwen_desc(), 1024)
    assert n == plain                       # bf16 look-ahead rows are read in place
    f32 = dict(act_dtype=bnd.TTT_F32, seq_len=4096)
    st, n = continue_ws(L, qwen_desc(**f32), 1024)
    _, plain = ws_size(L, qwen_desc(**f32), 1024)
    extra = 3 * 2560 * 2                    # K - 1 rows cast to bf16
    assert st == OK and plain + extra <= n <= plain + extra + 256


def continue_fwd(L, desc, p, x0n, n_next, ws_bytes=1 << 62, eta=1e-3):
    # H, X0, X0_next, n_next, Wg, Wu, W_state, taps, W_target, eta, chunk, O, ws
    return L.ttt_layer_forward_continue(ctypes.byref(desc), p[0], p[1], x0n, n_next, p[2],
                                        p[3], p[4], p[5], p[6], ctypes.c_float(eta), 1024,
                                        p[7], p[9], ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("n_next,code", [(-1, INVALID), (4, INVALID), (64, INVALID)])
def test_continue_rejects_lookahead_count(L, n_next, code):
    p = good_ptrs()
    assert continue_fwd(L, qwen_desc(), p, p[8], n_next) == code


def test_continue_validates_before_launch(L):
    p = good_ptrs()
    # X0_next is required when rows are promised, not when n_next is 0
    assert continue_fwd(L, qwen_desc(), p, None, 3) == INVALID
    # the state layout is fixed: no W_down0 stride
    assert continue_fwd(L, qwen_desc(w0_batch_stride=2560 * 9728), p, p[8], 3) == INVALID
    # NULL / misaligned state
    q = list(p)
    q[4] = None
    assert continue_fwd(L, qwen_desc(), q, p[8], 3) == INVALID
    q[4] = ctypes.c_void_p(p[4].value + 4)
    assert continue_fwd(L, qwen_desc(), q, p[8], 3) == INVALID
    # the in-place state may not overlap an input or the other outputs
    q = list(p)
    q[4] = p[1]
    assert continue_fwd(L, qwen_desc(), q, p[8], 3) == ALIAS
    assert continue_fwd(L, qwen_desc(), p, p[4], 3) == ALIAS     # X0_next is the state
    assert continue_fwd(L, qwen_desc(), p, p[7], 3) == ALIAS     # X0_next is O
    assert continue_fwd(L, qwen_desc(), p, p[8], 3, eta=float("nan")) == INVALID
    _, need = continue_ws(L, qwen_desc(), 1024)
    assert continue_fwd(L, qwen_desc(), p, p[8], 3, ws_bytes=need - 1) == WORKSPACE
    assert continue_fwd(L, qwen_desc(), p, None, 0, ws_bytes=need - 1) == WORKSPACE


# ---- decode --------------------------------------------------------------------

def decode_desc(**kw):
    a = dict(batch=1, seq_len=1, d_model=2560, d_ff=9728, conv_k=4, flags=bnd.FLAG_PAD_CHUNK)
    a.update(kw)
    return bnd.make_desc(**a)


def decode_size(L, desc, chunk=1024):
    n = ctypes.c_size_t(0)
    st = L.ttt_decode_state_size(ctypes.byref(desc), chunk, ctypes.byref(n))
    return st, n.value


def test_decode_state_size(L):
    st, n = decode_size(L, decode_desc(batch=2))
    assert st == OK, L.ttt_last_error()
    B, d, f, C = 2, 2560, 9728, 1024

    def pad(x):
        return x + 64 if (x // 64) % 2 == 0 else x
    ld_y = pad(d)
    expect = (B * d * f * 2            # bf16 copies of the states (d rows: whole 256-row slabs)
              + B * f * C * 2          # the open chunk's Z^T (f rows: whole slabs)
              + B * C * d * 2          # the open chunk's X0 rows
              + B * f * 2                      # z (bf16, the apply's operand)
              + B * C * ld_y * 2 + d * ld_y * 2 + B * d * C * 2   # Y, W_target^T, V^T
              + B * C * f * 4          # the open chunk's fp32 Z rows (fp16 range repair)
              + 4 * 256 * 4)           # the range buffer
    expect += B * ((-(-f // 256) * 256) - f) * C * 2   # f's last slab is whole
    assert expect <= n <= expect + 11 * 256


@pytest.mark.parametrize("kw,code", [
    (dict(flags=0), UNSUPPORTED),                       # sequence padding
    (dict(seq_len=2), INVALID),                         # one token per step
    (dict(w0_batch_stride=2560 * 9728), INVALID),       # W_state is [B, d, f]
    (dict(conv_k=0), INVALID)])
def test_decode_descriptor_checks(L, kw, code):
    st, _ = decode_size(L, decode_desc(**kw))
    assert st == code, (kw, st, L.ttt_last_error())


def decode_step(L, desc, p, pos=0, eta=1e-3, bytes_=1 << 62):
    # h, x0, Wg, Wu, taps, W_target, eta, chunk, pos, W_state, dstate, bytes, o
    return L.ttt_decode_step(ctypes.byref(desc), p[0], p[1], p[2], p[3], p[4], p[5],
                             ctypes.c_float(eta), 1024, pos, p[6], p[9],
                             ctypes.c_size_t(bytes_), p[7], None)


def test_decode_step_validates_before_launch(L):
    p = good_ptrs()
    desc = decode_desc()
    assert decode_step(L, desc, p, pos=-1) == INVALID
    assert decode_step(L, desc, p, eta=float("nan")) == INVALID
    _, need = decode_size(L, desc)
    assert decode_step(L, desc, p, bytes_=need - 1) == WORKSPACE
    q = list(p)
    q[7] = p[0]                                         # o is h
    assert decode_step(L, desc, q) == ALIAS
    q = list(p)
    q[6] = p[2]                                         # W_state is Wg
    assert decode_step(L, desc, q) == ALIAS
    q = list(p)
    q[6] = None
    assert decode_step(L, desc, q) == INVALID
    assert L.ttt_decode_begin(ctypes.byref(desc), 1024, p[6], p[9], ctypes.c_size_t(need - 1),
                              None) == WORKSPACE
    assert L.ttt_decode_begin(ctypes.byref(decode_desc(flags=0)), 1024, p[6], p[9],
                              ctypes.c_size_t(1 << 62), None) == UNSUPPORTED


# ---- the backward pass ------------------------------------------------------

def bwd_ws(L, desc, chunk=1024):
    n = ctypes.c_size_t(0)
    st = L.ttt_backward_workspace_size(ctypes.byref(desc), chunk, ctypes.byref(n))
    return st, n.value


def test_backward_workspace_size(L):
    st, n = bwd_ws(L, qwen_desc())
    assert st == OK
    B, T, d, f, k = 1, 65536, 2560, 9728, 64
    # at least the per-chunk bf16 states W_i^T and state gradients (both
    # halves of [W_i^T | Gbar^T], and Gbar itself), Z, Z^T, the SiLU factors
    # (fp32 words), [dG | dU] token-major, dG^T and dU^T
    floor = 3 * k * d * f * 2 + B * T * f * (2 + 2 + 4 + 2 * 2 + 2 + 2)
    assert floor <= n <= floor * 3 // 2
    st2, n2 = bwd_ws(L, qwen_desc(batch=2, w0_batch_stride=2560 * 9728))
    assert st2 == OK and n2 > n
    assert bwd_ws(L, qwen_desc(), 100)[0] == UNSUPPORTED


def backward(L, desc, p, dwf=True, eta=1e-3, chunk=1024, ws_bytes=1 << 62):
    """p: the seven inputs, dO, dW_final, the seven outputs, the workspace."""
    return L.ttt_layer_backward(ctypes.byref(desc), *p[:7], ctypes.c_float(eta), chunk, p[7],
                                p[8] if dwf else None, *p[9:16], p[16],
                                ctypes.c_size_t(ws_bytes), None)


def test_backward_validates_before_launch(L):
    fb = FakeBuffers()
    p = [fb[i] for i in range(17)]
    desc = qwen_desc()
    assert backward(L, desc, p, eta=float("nan")) == INVALID
    for i in list(range(8)) + list(range(9, 17)):
        q = list(p)
        q[i] = ctypes.c_void_p(0)
        assert backward(L, desc, q) == INVALID, i
        assert "NULL" in L.ttt_last_error().decode()
    q = list(p)
    q[8] = ctypes.c_void_p(p[8].value + 2)            # dW_final misaligned
    assert backward(L, desc, q) == INVALID
    _, need = bwd_ws(L, desc)
    assert backward(L, desc, p, ws_bytes=need - 1) == WORKSPACE
    q = list(p)
    q[9] = ctypes.c_void_p(p[0].value + 4096)         # dH inside H
    assert backward(L, desc, q) == ALIAS
    q = list(p)
    q[15] = ctypes.c_void_p(p[16].value + 4096)       # dW_target inside the workspace
    assert backward(L, desc, q) == ALIAS
    # per-sequence W_down0 at a stride other than d_model * d_ff
    assert backward(L, qwen_desc(batch=2, w0_batch_stride=2 * 2560 * 9728), p) == UNSUPPORTED
    assert "stride" in L.ttt_last_error().decode()


# ---- training: the forward that keeps its activations, and its backward ----

def train_sizes(L, desc, chunk=1024):
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st1 = L.ttt_train_workspace_size(ctypes.byref(desc), chunk, ctypes.byref(a))
    st2 = L.ttt_backward_saved_workspace_size(ctypes.byref(desc), chunk, ctypes.byref(b))
    return st1, a.value, st2, b.value


def test_train_workspace_sizes(L):
    desc = qwen_desc()
    st1, fwd_train, st2, bwd_saved = train_sizes(L, desc)
    assert st1 == OK and st2 == OK
    _, fwd = ws_size(L, desc, 1024)
    _, bwd = bwd_ws(L, desc)
    B, T, d, f = 1, 65536, 2560, 9728
    # the training forward keeps a bf16 Z^T and the SiLU factors besides
    assert fwd_train - fwd >= B * T * f * (2 + 4)
    # the saved backward needs no Z, Z^T, SiLU factors or packed weights
    assert bwd - bwd_saved >= B * T * f * (2 + 2 + 4)
    running = qwen_desc(flags=bnd.FLAG_SCHED_RUNNING)
    st1, _, st2, _ = train_sizes(L, running)
    assert st1 == UNSUPPORTED and st2 == UNSUPPORTED
    assert "prefix" in L.ttt_last_error().decode()


def test_train_entry_points_validate_before_launch(L):
    fb = FakeBuffers()
    p = [fb[i] for i in range(18)]
    desc = qwen_desc()
    st1, need_fwd, _, need_bwd = train_sizes(L, desc)
    st = L.ttt_layer_forward_train(ctypes.byref(desc), *p[:7], ctypes.c_float(1e-3), 1024, p[7],
                                   p[8], p[9], ctypes.c_size_t(need_fwd - 1), None)
    assert st == WORKSPACE
    st = L.ttt_layer_forward_train(ctypes.byref(qwen_desc(flags=bnd.FLAG_SCHED_RUNNING)),
                                   *p[:7], ctypes.c_float(1e-3), 1024, p[7], p[8], p[9],
                                   ctypes.c_size_t(1 << 62), None)
    assert st == UNSUPPORTED

    def bwd(saved, saved_bytes, ws_bytes=1 << 62):
        return L.ttt_layer_backward_saved(ctypes.byref(desc), *p[:7], ctypes.c_float(1e-3), 1024,
                                          saved, ctypes.c_size_t(saved_bytes), p[8], p[9],
                                          *p[10:17], p[17], ctypes.c_size_t(ws_bytes), None)
    assert bwd(ctypes.c_void_p(0), need_fwd) == INVALID
    assert bwd(p[7], need_fwd - 1) == WORKSPACE
    assert "saved" in L.ttt_last_error().decode()
    assert bwd(p[7], need_fwd, ws_bytes=need_bwd - 1) == WORKSPACE
    q = list(p)
    q[10] = ctypes.c_void_p(p[7].value + 4096)        # dH inside saved
    st = L.ttt_layer_backward_saved(ctypes.byref(desc), *q[:7], ctypes.c_float(1e-3), 1024,
                                    q[7], ctypes.c_size_t(need_fwd), q[8], q[9], *q[10:17],
                                    q[17], ctypes.c_size_t(1 << 62), None)
    assert st == ALIAS


# ---- the no-allocation entry point ------------------------------------------

def test_noalloc_rejects_problems_beyond_its_scratch(L):
    """A workload whose workspace exceeds the static scratch is refused with
    TTT_ERR_WORKSPACE on the host, before any HIP call (this runs without a
    GPU)."""
    p = good_ptrs()
    desc = qwen_desc()
    st = L.ttt_layer_forward_noalloc(ctypes.byref(desc), *p[:7], ctypes.c_float(1e-3), 1024,
                                     p[7], p[8], None)
    assert st == WORKSPACE
    msg = L.ttt_last_error().decode()
    assert "static scratch" in msg and str(64 << 20) in msg
    desc = qwen_desc(batch=0)
    st = L.ttt_layer_forward_noalloc(ctypes.byref(desc), *p[:7], ctypes.c_float(1e-3), 1024,
                                     p[7], p[8], None)
    assert st == INVALID
