"""ctypes marshalling for libttt_layer.so (C ABI: include/ttt.h).

Only argument checking and marshalling live here: tensors are passed to the
library as raw device pointers, together with torch's current HIP stream.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttt_layer.so")

TTT_BF16, TTT_F32 = 0, 1
FLAG_PAD_CHUNK = 1 << 0
FLAG_SCHED_RUNNING = 1 << 1
FLAG_SCHED_PREFIX = 1 << 2


class TTTError(RuntimeError):
    """A non-OK status from libttt_layer, with its name and message."""

    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("conv_k", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("w0_batch_stride", ctypes.c_int64), ("flags", ctypes.c_uint32),
                ("reserved2", ctypes.c_uint32)]


class PackedBlock(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("doc_end", ctypes.c_int32), ("chunk_end", ctypes.c_int32)]


class PackedTile(ctypes.Structure):
    _fields_ = [("t0", ctypes.c_int32), ("t1", ctypes.c_int32),
                ("snapshot", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


_lib = None
_P = ctypes.c_void_p
_S = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libttt_layer.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m test_layer_gate_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    DP = ctypes.POINTER(Desc)
    L.ttt_workspace_size.argtypes = [DP, ctypes.c_int32, ctypes.POINTER(_S)]
    L.ttt_step_workspace_size.argtypes = [DP, ctypes.POINTER(_S)]
    L.ttt_layer_forward.argtypes = [DP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                    ctypes.c_int32, _P, _P, _P, _S, _P]
    I32P = ctypes.POINTER(ctypes.c_int32)
    L.ttt_clipped_workspace_size.argtypes = [DP, ctypes.c_int32, ctypes.c_float,
                                             ctypes.POINTER(_S)]
    L.ttt_layer_forward_clipped.argtypes = [DP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                            ctypes.c_int32, ctypes.c_float, _P, _P, _P, _S, _P]
    L.ttt_packed_workspace_size.argtypes = [DP, ctypes.c_int32, I32P, ctypes.c_int32,
                                            ctypes.POINTER(_S)]
    L.ttt_layer_forward_packed.argtypes = [DP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                           ctypes.c_int32, I32P, ctypes.c_int32, _P, _P, _P,
                                           _S, _P]
    L.ttt_packed_clipped_workspace_size.argtypes = [DP, ctypes.c_int32, I32P, ctypes.c_int32,
                                                    ctypes.c_float, ctypes.POINTER(_S)]
    L.ttt_layer_forward_packed_clipped.argtypes = [DP, _P, _P, _P, _P, _P, _P, _P,
                                                   ctypes.c_float, ctypes.c_int32, I32P,
                                                   ctypes.c_int32, ctypes.c_float, _P, _P, _P,
                                                   _S, _P]
    L.ttt_packed_tables.argtypes = [DP, ctypes.c_int32, I32P, ctypes.c_int32,
                                    ctypes.POINTER(PackedBlock), ctypes.c_int32,
                                    ctypes.POINTER(PackedTile), ctypes.c_int32, I32P]
    L.ttt_continue_workspace_size.argtypes = [DP, ctypes.c_int32, ctypes.POINTER(_S)]
    L.ttt_layer_forward_continue.argtypes = [DP, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P,
                                             _P, ctypes.c_float, ctypes.c_int32, _P, _P, _S,
                                             _P]
    L.ttt_decode_state_size.argtypes = [DP, ctypes.c_int32, ctypes.POINTER(_S)]
    L.ttt_decode_begin.argtypes = [DP, ctypes.c_int32, _P, _P, _S, _P]
    L.ttt_decode_step.argtypes = [DP, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int32,
                                  ctypes.c_int32, _P, _P, _S, _P, _P]
    L.ttt_layer_forward_noalloc.argtypes = [DP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                            ctypes.c_int32, _P, _P, _P]
    L.ttt_backward_workspace_size.argtypes = [DP, ctypes.c_int32, ctypes.POINTER(_S)]
    L.ttt_train_workspace_size.argtypes = [DP, ctypes.c_int32, ctypes.POINTER(_S)]
    L.ttt_backward_saved_workspace_size.argtypes = [DP, ctypes.c_int32, ctypes.POINTER(_S)]
    L.ttt_layer_forward_train.argtypes = [DP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                          ctypes.c_int32, _P, _P, _P, _S, _P]
    L.ttt_layer_backward_saved.argtypes = [DP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                           ctypes.c_int32, _P, _S, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _S, _P]
    L.ttt_layer_backward.argtypes = [DP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                     ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _S, _P]
    L.ttt_gated_activation.argtypes = [DP, _P, _P, _P, _P, _P, _S, _P]
    L.ttt_lm_target.argtypes = [DP, _P, _P, _P, ctypes.c_int32, _P, _P, _S, _P]
    for fn in ("ttt_workspace_size", "ttt_step_workspace_size", "ttt_layer_forward",
               "ttt_layer_forward_noalloc",
               "ttt_packed_workspace_size", "ttt_layer_forward_packed",
               "ttt_clipped_workspace_size", "ttt_layer_forward_clipped",
               "ttt_packed_clipped_workspace_size", "ttt_layer_forward_packed_clipped",
               "ttt_packed_tables",
               "ttt_continue_workspace_size", "ttt_layer_forward_continue",
               "ttt_decode_state_size", "ttt_decode_begin", "ttt_decode_step",
               "ttt_backward_workspace_size", "ttt_layer_backward",
               "ttt_train_workspace_size", "ttt_layer_forward_train",
               "ttt_backward_saved_workspace_size", "ttt_layer_backward_saved",
               "ttt_gated_activation", "ttt_lm_target", "ttt_profile_enable"):
        getattr(L, fn).restype = ctypes.c_int
    L.ttt_status_string.argtypes = [ctypes.c_int32]
    L.ttt_status_string.restype = ctypes.c_char_p
    L.ttt_last_error.argtypes = []
    L.ttt_last_error.restype = ctypes.c_char_p
    L.ttt_profile_enable.argtypes = [ctypes.c_int32]
    L.ttt_copy_calibration.argtypes = [_P, _P, _S, _P]
    L.ttt_copy_calibration.restype = ctypes.c_int
    L.ttt_profile_read.argtypes = [ctypes.POINTER(KernelStat), ctypes.c_int32]
    L.ttt_profile_read.restype = ctypes.c_int32
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise TTTError(status, L.ttt_status_string(status).decode(),
                       L.ttt_last_error().decode())


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype == torch.bfloat16:
        return TTT_BF16
    if t.dtype == torch.float32:
        return TTT_F32
    raise TypeError(f"{what} must be bfloat16 or float32, got {t.dtype}")


def make_desc(batch, seq_len, d_model, d_ff, conv_k, act_dtype=TTT_BF16,
              weight_dtype=TTT_BF16, w0_batch_stride=0, flags=0) -> Desc:
    return Desc(batch, seq_len, d_model, d_ff, conv_k, act_dtype, weight_dtype, 0,
                w0_batch_stride, flags, 0)


def _flags(schedule, pad):
    fl = 0
    if pad == "chunk":
        fl |= FLAG_PAD_CHUNK
    elif pad != "sequence":
        raise ValueError(f"pad must be 'sequence' or 'chunk', got {pad!r}")
    if schedule == "running":
        fl |= FLAG_SCHED_RUNNING
    elif schedule == "prefix":
        fl |= FLAG_SCHED_PREFIX
    elif schedule is not None:
        raise ValueError(f"schedule must be None, 'prefix' or 'running', got {schedule!r}")
    return fl


def _require_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def workspace_size(desc: Desc, chunk: int) -> int:
    n = _S(0)
    _check(lib().ttt_workspace_size(ctypes.byref(desc), chunk, ctypes.byref(n)))
    return n.value


def clipped_workspace_size(desc: Desc, chunk: int, clip: float) -> int:
    n = _S(0)
    _check(lib().ttt_clipped_workspace_size(ctypes.byref(desc), int(chunk),
                                            ctypes.c_float(float(clip)), ctypes.byref(n)))
    return n.value


def _layer_desc(H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, schedule, pad):
    """The descriptor of a prefill call, after checking shapes and dtypes."""
    _require_cuda(H, X0, Wg, Wu, W_down0, conv_taps, W_target)
    if H.dim() != 3 or X0.shape != H.shape:
        raise ValueError("H and X0 must both be [B, T, d]")
    B, T, d = H.shape
    f = Wg.shape[0]
    K = conv_taps.shape[0]
    if Wg.shape != (f, d) or Wu.shape != (f, d):
        raise ValueError("Wg and Wu must be [d_ff, d_model]")
    if W_down0.shape not in ((d, f), (B, d, f)):
        raise ValueError("W_down0 must be [d_model, d_ff] or [B, d_model, d_ff]")
    if conv_taps.shape != (K, d) or W_target.shape != (d, d):
        raise ValueError("conv_taps must be [K, d_model] and W_target [d_model, d_model]")
    act = _dtype_code(H, "H")
    wt = _dtype_code(Wg, "Wg")
    if X0.dtype != H.dtype:
        raise TypeError("X0 must have H's dtype")
    for t, n in ((Wu, "Wu"), (W_down0, "W_down0"), (conv_taps, "conv_taps"),
                 (W_target, "W_target")):
        if t.dtype != Wg.dtype:
            raise TypeError(f"{n} must have Wg's dtype")
    if not math.isfinite(float(eta)):
        raise ValueError("eta must be finite")
    stride = d * f if W_down0.dim() == 3 else 0
    return make_desc(B, T, d, f, K, act, wt, stride, _flags(schedule, pad))


def layer_forward(H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, chunk, *,
                  schedule=None, pad="sequence", clip=None, out=None, W_down_final=None,
                  workspace=None, stream=None):
    """O, W_final for H, X0 [B, T, d]; Wg, Wu [f, d]; W_down0 [d, f] or
    [B, d, f]; conv_taps [K, d]; W_target [d, d] (see include/ttt.h).

    schedule: None (library default), "prefix" or "running". pad:
    "sequence" (conv reads zero past the sequence end) or "chunk". clip:
    None, or the Frobenius-norm limit of every chunk's update
    (ttt_layer_forward_clipped).
    """
    desc = _layer_desc(H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, schedule, pad)
    B, T, d = H.shape
    f = Wg.shape[0]
    if clip is None:
        ws_bytes = workspace_size(desc, int(chunk))
    else:
        ws_bytes = clipped_workspace_size(desc, int(chunk), clip)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=H.device)
    O = torch.empty_like(H) if out is None else out
    Wf = (torch.empty((B, d, f), dtype=torch.float32, device=H.device)
          if W_down_final is None else W_down_final)
    _require_cuda(O, Wf, workspace)
    args = [ctypes.byref(desc), _ptr(H), _ptr(X0), _ptr(Wg), _ptr(Wu), _ptr(W_down0),
            _ptr(conv_taps), _ptr(W_target), ctypes.c_float(float(eta)), int(chunk)]
    tail = [_ptr(O), _ptr(Wf), _ptr(workspace), workspace.numel(), _stream(stream)]
    if clip is None:
        _check(lib().ttt_layer_forward(*args, *tail))
    else:
        _check(lib().ttt_layer_forward_clipped(*args, ctypes.c_float(float(clip)), *tail))
    return O, Wf


def backward_workspace_size(desc: Desc, chunk: int) -> int:
    n = _S(0)
    _check(lib().ttt_backward_workspace_size(ctypes.byref(desc), int(chunk), ctypes.byref(n)))
    return n.value


def train_workspace_size(desc: Desc, chunk: int) -> int:
    n = _S(0)
    _check(lib().ttt_train_workspace_size(ctypes.byref(desc), int(chunk), ctypes.byref(n)))
    return n.value


def backward_saved_workspace_size(desc: Desc, chunk: int) -> int:
    n = _S(0)
    _check(lib().ttt_backward_saved_workspace_size(ctypes.byref(desc), int(chunk),
                                                   ctypes.byref(n)))
    return n.value


def layer_forward_train(H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, chunk, *,
                        pad="sequence", out=None, W_down_final=None, workspace=None,
                        stream=None):
    """ttt_layer_forward_train: the prefill (prefix schedule) that keeps in its
    workspace what the backward reads. Returns O, W_final and that workspace,
    to pass unchanged to layer_backward(..., saved=...)."""
    desc = _layer_desc(H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, None, pad)
    B, T, d = H.shape
    f = Wg.shape[0]
    ws_bytes = train_workspace_size(desc, int(chunk))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=H.device)
    O = torch.empty_like(H) if out is None else out
    Wf = (torch.empty((B, d, f), dtype=torch.float32, device=H.device)
          if W_down_final is None else W_down_final)
    _require_cuda(O, Wf, workspace)
    _check(lib().ttt_layer_forward_train(
        ctypes.byref(desc), _ptr(H), _ptr(X0), _ptr(Wg), _ptr(Wu), _ptr(W_down0),
        _ptr(conv_taps), _ptr(W_target), ctypes.c_float(float(eta)), int(chunk), _ptr(O),
        _ptr(Wf), _ptr(workspace), workspace.numel(), _stream(stream)))
    return O, Wf, workspace


def layer_backward(H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, chunk, dO, *,
                   dW_final=None, pad="sequence", saved=None, out=None, workspace=None,
                   stream=None):
    """The prefill's gradients (ttt_layer_backward) for the upstream
    gradients dO [B, T, d] (H's dtype) and dW_final [B, d, f] fp32 (None:
    zero). Returns a dict of fp32 tensors: dH, dX0 [B, T, d]; dWg, dWu
    [f, d]; dW_down0 [d, f] (shared W_down0) or [B, d, f]; dtaps [K, d];
    dW_target [d, d]. out: such a dict to write into instead of new tensors.
    saved: the workspace layer_forward_train returned for the same arguments
    (ttt_layer_backward_saved: no recompute of gate/up and the states)."""
    desc = _layer_desc(H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, None, pad)
    B, T, d = H.shape
    f, K = Wg.shape[0], conv_taps.shape[0]
    _require_cuda(dO)
    if dO.shape != H.shape or dO.dtype != H.dtype:
        raise ValueError("dO must be [B, T, d] with H's dtype")
    if dW_final is not None:
        _require_cuda(dW_final)
        if dW_final.shape != (B, d, f) or dW_final.dtype != torch.float32:
            raise ValueError("dW_final must be [B, d_model, d_ff] float32")
        if not dW_final.is_contiguous():
            raise ValueError("dW_final must be contiguous")
    if saved is not None:
        _require_cuda(saved)
        ws_bytes = backward_saved_workspace_size(desc, int(chunk))
    else:
        ws_bytes = backward_workspace_size(desc, int(chunk))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=H.device)
    _require_cuda(workspace)
    shapes = {"dH": (B, T, d), "dX0": (B, T, d), "dWg": (f, d), "dWu": (f, d),
              "dW_down0": tuple(W_down0.shape), "dtaps": (K, d), "dW_target": (d, d)}
    if out is None:
        g = {k: torch.empty(v, dtype=torch.float32, device=H.device) for k, v in shapes.items()}
    else:
        g = out
        for k, v in shapes.items():
            if k not in g or tuple(g[k].shape) != v or g[k].dtype != torch.float32:
                raise ValueError(f"out[{k!r}] must be a float32 tensor of shape {v}")
            _require_cuda(g[k])
    head = [ctypes.byref(desc), _ptr(H), _ptr(X0), _ptr(Wg), _ptr(Wu), _ptr(W_down0),
            _ptr(conv_taps), _ptr(W_target), ctypes.c_float(float(eta)), int(chunk)]
    tail = [_ptr(dO), None if dW_final is None else _ptr(dW_final),
            _ptr(g["dH"]), _ptr(g["dX0"]), _ptr(g["dWg"]), _ptr(g["dWu"]), _ptr(g["dW_down0"]),
            _ptr(g["dtaps"]), _ptr(g["dW_target"]), _ptr(workspace), workspace.numel(),
            _stream(stream)]
    if saved is None:
        _check(lib().ttt_layer_backward(*head, *tail))
    else:
        _check(lib().ttt_layer_backward_saved(*head, _ptr(saved), saved.numel(), *tail))
    return g


def _doc_array(doc_starts):
    starts = [int(v) for v in doc_starts]
    return (ctypes.c_int32 * max(len(starts), 1))(*starts), len(starts)


def packed_workspace_size(desc: Desc, chunk: int, doc_starts, clip=None) -> int:
    arr, n_docs = _doc_array(doc_starts)
    n = _S(0)
    if clip is None:
        _check(lib().ttt_packed_workspace_size(ctypes.byref(desc), chunk, arr, n_docs,
                                               ctypes.byref(n)))
    else:
        _check(lib().ttt_packed_clipped_workspace_size(ctypes.byref(desc), chunk, arr, n_docs,
                                                       ctypes.c_float(float(clip)),
                                                       ctypes.byref(n)))
    return n.value


def layer_forward_packed(H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, chunk,
                         doc_starts, *, schedule=None, pad="sequence", clip=None, out=None,
                         W_down_final=None, workspace=None, stream=None):
    """O, W_final for one packed sequence of documents (include/ttt.h,
    ttt_layer_forward_packed). H, X0 [T, d] or [1, T, d]; doc_starts: the
    documents' first tokens, increasing from 0, multiples of 64. clip: None
    or each chunk's update-norm limit (ttt_layer_forward_packed_clipped). O
    has H's shape; W_final is [d, f] (or [1, d, f] for 3-D H): the state
    after the last document."""
    _require_cuda(H, X0, Wg, Wu, W_down0, conv_taps, W_target)
    squeeze = H.dim() == 2
    H3 = H.unsqueeze(0) if squeeze else H
    X3 = X0.unsqueeze(0) if X0.dim() == 2 else X0
    if H3.dim() != 3 or H3.shape[0] != 1 or X3.shape != H3.shape:
        raise ValueError("H and X0 must both be [T, d] or [1, T, d]")
    _, T, d = H3.shape
    f = Wg.shape[0]
    K = conv_taps.shape[0]
    if Wg.shape != (f, d) or Wu.shape != (f, d) or W_down0.shape != (d, f):
        raise ValueError("Wg, Wu must be [d_ff, d_model] and W_down0 [d_model, d_ff]")
    if conv_taps.shape != (K, d) or W_target.shape != (d, d):
        raise ValueError("conv_taps must be [K, d_model] and W_target [d_model, d_model]")
    act = _dtype_code(H3, "H")
    wt = _dtype_code(Wg, "Wg")
    if X3.dtype != H3.dtype:
        raise TypeError("X0 must have H's dtype")
    for t, n in ((Wu, "Wu"), (W_down0, "W_down0"), (conv_taps, "conv_taps"),
                 (W_target, "W_target")):
        if t.dtype != Wg.dtype:
            raise TypeError(f"{n} must have Wg's dtype")
    if not math.isfinite(float(eta)):
        raise ValueError("eta must be finite")
    desc = make_desc(1, T, d, f, K, act, wt, 0, _flags(schedule, pad))
    arr, n_docs = _doc_array(doc_starts)
    ws_bytes = packed_workspace_size(desc, int(chunk), doc_starts, clip)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=H.device)
    O = torch.empty_like(H3) if out is None else out.view(1, T, d)
    Wf = (torch.empty((1, d, f), dtype=torch.float32, device=H.device)
          if W_down_final is None else W_down_final.view(1, d, f))
    _require_cuda(O, Wf, workspace)
    args = (ctypes.byref(desc), _ptr(H3), _ptr(X3), _ptr(Wg), _ptr(Wu), _ptr(W_down0),
            _ptr(conv_taps), _ptr(W_target), ctypes.c_float(float(eta)), int(chunk), arr, n_docs)
    tail = (_ptr(O), _ptr(Wf), _ptr(workspace), workspace.numel(), _stream(stream))
    if clip is None:
        _check(lib().ttt_layer_forward_packed(*args, *tail))
    else:
        _check(lib().ttt_layer_forward_packed_clipped(*args, ctypes.c_float(float(clip)),
                                                      *tail))
    return (O[0], Wf[0]) if squeeze else (O, Wf)


def packed_tables(desc: Desc, chunk: int, doc_starts):
    """The block table and apply tiles ttt_layer_forward_packed builds for a
    layout (include/ttt.h, ttt_packed_tables; host only): (blocks, tiles,
    n_chunks), blocks as (chunk, flags, doc_end, chunk_end) tuples and tiles
    as (t0, t1, snapshot) tuples."""
    arr, n_docs = _doc_array(doc_starts)
    counts = (ctypes.c_int32 * 3)()
    _check(lib().ttt_packed_tables(ctypes.byref(desc), int(chunk), arr, n_docs, None, 0, None,
                                   0, counts))
    nb, nt = counts[0], counts[1]
    blocks = (PackedBlock * max(nb, 1))()
    tiles = (PackedTile * max(nt, 1))()
    _check(lib().ttt_packed_tables(ctypes.byref(desc), int(chunk), arr, n_docs, blocks, nb,
                                   tiles, nt, counts))
    return ([(b.chunk, b.flags, b.doc_end, b.chunk_end) for b in blocks[:nb]],
            [(t.t0, t.t1, t.snapshot) for t in tiles[:nt]], counts[2])


def continue_workspace_size(desc: Desc, chunk: int) -> int:
    n = _S(0)
    _check(lib().ttt_continue_workspace_size(ctypes.byref(desc), chunk, ctypes.byref(n)))
    return n.value


def layer_forward_continue(H, X0, X0_next, Wg, Wu, W_state, conv_taps, W_target, eta,
                           chunk, *, schedule=None, pad="sequence", out=None,
                           workspace=None, stream=None):
    """O for the next segment of B sequences (include/ttt.h,
    ttt_layer_forward_continue). H, X0 [B, T, d]; X0_next [B, L, d] with
    0 <= L <= K - 1 (the X0 rows that follow the segment), or None; W_state
    [B, d, f] float32, read as the state before the segment and overwritten
    in place with the state after it. Returns O."""
    _require_cuda(H, X0, Wg, Wu, W_state, conv_taps, W_target)
    if H.dim() != 3 or X0.shape != H.shape:
        raise ValueError("H and X0 must both be [B, T, d]")
    B, T, d = H.shape
    f = Wg.shape[0]
    K = conv_taps.shape[0]
    if Wg.shape != (f, d) or Wu.shape != (f, d):
        raise ValueError("Wg and Wu must be [d_ff, d_model]")
    if W_state.shape != (B, d, f) or W_state.dtype != torch.float32:
        raise ValueError("W_state must be float32 [B, d_model, d_ff]")
    if conv_taps.shape != (K, d) or W_target.shape != (d, d):
        raise ValueError("conv_taps must be [K, d_model] and W_target [d_model, d_model]")
    act = _dtype_code(H, "H")
    wt = _dtype_code(Wg, "Wg")
    if X0.dtype != H.dtype:
        raise TypeError("X0 must have H's dtype")
    for t, n in ((Wu, "Wu"), (conv_taps, "conv_taps"), (W_target, "W_target")):
        if t.dtype != Wg.dtype:
            raise TypeError(f"{n} must have Wg's dtype")
    n_next = 0
    if X0_next is not None:
        _require_cuda(X0_next)
        if X0_next.dim() != 3 or X0_next.shape[0] != B or X0_next.shape[2] != d:
            raise ValueError("X0_next must be [B, L, d]")
        if X0_next.dtype != H.dtype:
            raise TypeError("X0_next must have H's dtype")
        n_next = X0_next.shape[1]
    if not math.isfinite(float(eta)):
        raise ValueError("eta must be finite")
    desc = make_desc(B, T, d, f, K, act, wt, 0, _flags(schedule, pad))
    ws_bytes = continue_workspace_size(desc, int(chunk))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=H.device)
    O = torch.empty_like(H) if out is None else out
    _require_cuda(O, workspace)
    _check(lib().ttt_layer_forward_continue(
        ctypes.byref(desc), _ptr(H), _ptr(X0),
        _ptr(X0_next) if n_next > 0 else ctypes.c_void_p(0), int(n_next), _ptr(Wg), _ptr(Wu),
        _ptr(W_state), _ptr(conv_taps), _ptr(W_target), ctypes.c_float(float(eta)),
        int(chunk), _ptr(O), _ptr(workspace), workspace.numel(), _stream(stream)))
    return O


def _decode_desc(h, Wg, conv_taps):
    B, d = h.shape
    return make_desc(B, 1, d, Wg.shape[0], conv_taps.shape[0], _dtype_code(h, "h"),
                     _dtype_code(Wg, "Wg"), 0, FLAG_PAD_CHUNK)


def decode_state_size(desc: Desc, chunk: int) -> int:
    n = _S(0)
    _check(lib().ttt_decode_state_size(ctypes.byref(desc), int(chunk), ctypes.byref(n)))
    return n.value


def decode_begin(W_state, chunk, decode_state, *, act_dtype=torch.bfloat16,
                 weight_dtype=torch.bfloat16, conv_k=1, stream=None):
    """Start decoding B sequences at a chunk boundary from W_state [B, d, f]
    float32 (include/ttt.h, ttt_decode_begin): writes the bf16 copy of the
    states into decode_state (uint8, decode_state_size bytes)."""
    _require_cuda(W_state, decode_state)
    if W_state.dim() != 3 or W_state.dtype != torch.float32:
        raise ValueError("W_state must be float32 [B, d_model, d_ff]")
    B, d, f = W_state.shape
    act = TTT_F32 if act_dtype == torch.float32 else TTT_BF16
    wt = TTT_F32 if weight_dtype == torch.float32 else TTT_BF16
    desc = make_desc(B, 1, d, f, conv_k, act, wt, 0, FLAG_PAD_CHUNK)
    _check(lib().ttt_decode_begin(ctypes.byref(desc), int(chunk), _ptr(W_state),
                                  _ptr(decode_state), decode_state.numel(), _stream(stream)))


def decode_step(h, x0, Wg, Wu, conv_taps, W_target, eta, chunk, pos, W_state, decode_state,
                *, out=None, stream=None):
    """One token per sequence (include/ttt.h, ttt_decode_step): h, x0 [B, d]
    at document position pos; W_state [B, d, f] float32 is updated in place
    when pos closes a chunk. Returns o [B, d]."""
    _require_cuda(h, x0, Wg, Wu, conv_taps, W_target, W_state, decode_state)
    if h.dim() != 2 or x0.shape != h.shape or x0.dtype != h.dtype:
        raise ValueError("h and x0 must both be [B, d_model] of one dtype")
    B, d = h.shape
    f = Wg.shape[0]
    if W_state.shape != (B, d, f) or W_state.dtype != torch.float32:
        raise ValueError("W_state must be float32 [B, d_model, d_ff]")
    for t, n in ((Wu, "Wu"), (conv_taps, "conv_taps"), (W_target, "W_target")):
        if t.dtype != Wg.dtype:
            raise TypeError(f"{n} must have Wg's dtype")
    if not math.isfinite(float(eta)):
        raise ValueError("eta must be finite")
    desc = _decode_desc(h, Wg, conv_taps)
    o = torch.empty_like(h) if out is None else out
    _require_cuda(o)
    _check(lib().ttt_decode_step(ctypes.byref(desc), _ptr(h), _ptr(x0), _ptr(Wg), _ptr(Wu),
                                 _ptr(conv_taps), _ptr(W_target), ctypes.c_float(float(eta)),
                                 int(chunk), int(pos), _ptr(W_state), _ptr(decode_state),
                                 decode_state.numel(), _ptr(o), _stream(stream)))
    return o


def _step_ws(desc, device):
    n = _S(0)
    _check(lib().ttt_step_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)


def gated_activation(H, Wg, Wu, *, stream=None):
    """Z = SiLU(H Wg^T) * (H Wu^T) in bf16, [B, T, d_ff]."""
    _require_cuda(H, Wg, Wu)
    B, T, d = H.shape
    f = Wg.shape[0]
    desc = make_desc(B, T, d, f, 1, _dtype_code(H, "H"), _dtype_code(Wg, "Wg"))
    ws = _step_ws(desc, H.device)
    Z = torch.empty((B, T, f), dtype=torch.bfloat16, device=H.device)
    _check(lib().ttt_gated_activation(ctypes.byref(desc), _ptr(H), _ptr(Wg), _ptr(Wu),
                                      _ptr(Z), _ptr(ws), ws.numel(), _stream(stream)))
    return Z


def lm_target(X0, conv_taps, W_target, *, chunk=64, pad="sequence", stream=None):
    """V = conv(X0) W_target in bf16, [B, T, d_model]."""
    _require_cuda(X0, conv_taps, W_target)
    B, T, d = X0.shape
    desc = make_desc(B, T, d, 64, conv_taps.shape[0], _dtype_code(X0, "X0"),
                     _dtype_code(conv_taps, "conv_taps"), 0, _flags(None, pad))
    ws = _step_ws(desc, X0.device)
    V = torch.empty((B, T, d), dtype=torch.bfloat16, device=X0.device)
    _check(lib().ttt_lm_target(ctypes.byref(desc), _ptr(X0), _ptr(conv_taps),
                               _ptr(W_target), int(chunk), _ptr(V), _ptr(ws),
                               ws.numel(), _stream(stream)))
    return V


def profile_enable(on: bool = True) -> None:
    _check(lib().ttt_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{kernel name: (launches, total ms)} for launches since profile_enable."""
    cap = 64
    arr = (KernelStat * cap)()
    n = min(lib().ttt_profile_read(arr, cap), cap)
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}


def copy_calibration(dst, src, *, stream=None):
    """dst <- src (same byte size, a multiple of 16) with the library's plain
    copy kernel, a known-size reference for hardware traffic counters."""
    _require_cuda(dst, src)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("dst and src must have the same size in bytes")
    _check(lib().ttt_copy_calibration(_ptr(dst), _ptr(src), n, _stream(stream)))
