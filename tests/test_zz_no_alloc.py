"""GPU: ttt_layer_forward_noalloc (the prefill with its workspace in the
library's static device scratch) against ttt_layer_forward with a caller
workspace, through the C ABI: the same kernels on the same inputs, so the
outputs must be identical bit for bit. Two calls in a row, the second with a
smaller problem, so that the second runs on the scratch the first left
behind; then the larger problem again."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from test_parity import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import test_layer_gate_amd as m
    m.lib()
    return m


def noalloc(ttt, t, eta, chunk, flags=0):
    from test_layer_gate_amd import _binding as bnd
    B, T, d = t["H"].shape
    f, K = t["Wg"].shape[0], t["taps"].shape[0]
    desc = bnd.make_desc(B, T, d, f, K, 0, 0, 0, flags)
    O = torch.full_like(t["H"], float("nan"))
    Wf = torch.full((B, d, f), float("nan"), dtype=torch.float32, device="cuda")
    p = [ctypes.c_void_p(x.data_ptr()) for x in
         (t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"], t["W_target"])]
    st = bnd.lib().ttt_layer_forward_noalloc(
        ctypes.byref(desc), *p, ctypes.c_float(eta), chunk, ctypes.c_void_p(O.data_ptr()),
        ctypes.c_void_p(Wf.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    bnd._check(st)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), Wf.cpu().numpy()


def plain(ttt, t, eta, chunk, **kw):
    O, Wf = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                              t["W_target"], eta, chunk, **kw)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), Wf.cpu().numpy()


def test_noalloc_equals_caller_workspace(ttt):
    big = synth.CONFIGS["mid_amp"]                       # T = 2048, d 256, f 1024
    small = synth.CONFIGS["tiny_amp"]                    # T = 256, d 64, f 256
    xb = to_dev(synth.make_inputs(big, batch=2, seed=5), big.dtype)
    xs = to_dev(synth.make_inputs(small, seq_len=200, seed=6), small.dtype)
    for t, cfg in ((xb, big), (xs, small), (xb, big)):
        print(f"[noalloc] B={t['H'].shape[0]} T={t['H'].shape[1]} d={cfg.d_model}", flush=True)
        Oa, Wa = noalloc(ttt, t, cfg.eta, cfg.chunk)
        Ob, Wb = plain(ttt, t, cfg.eta, cfg.chunk)
        assert np.array_equal(Oa, Ob) and np.array_equal(Wa, Wb)
    # the running schedule through the same scratch
    Oa, Wa = noalloc(ttt, xs, small.eta, small.chunk, flags=2)
    Ob, Wb = plain(ttt, xs, small.eta, small.chunk, schedule="running")
    assert np.array_equal(Oa, Ob) and np.array_equal(Wa, Wb)
