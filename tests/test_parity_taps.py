"""GPU parity over the conv's kernel size K, which the ABI takes from 1 to
64 (the configurations use 3 and 4; the pages' own example uses 5). The
conv kernel keeps a window of 8 X0 rows that slides one row per tap, so
K = 1, 8, 9 and 64 cover a window used partly, exactly, past one window and
at the limit. Checked against the CPU oracle with both paddings, and for a
continued segment with its K - 1 look-ahead rows. Tolerances as in
test_parity.py (amplified distributions, so the update is a large part of
the output).
"""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as ora
import synth
from test_parity import DW_TOL, O_TOL, rel, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import test_layer_gate_amd as m
    m.lib()
    return m


BASE = synth.CONFIGS["mid_amp"]


@pytest.mark.parametrize("pad", ["sequence", "chunk"])
@pytest.mark.parametrize("K", [1, 2, 5, 8, 9, 64])
def test_kernel_sizes_match_oracle(ttt, K, pad):
    # taps std 1/sqrt(K) keeps the target's magnitude independent of K
    cfg = BASE.with_(name=f"taps{K}", seq_len=700, chunk=128, conv_k=K,
                     taps_std=float(K) ** -0.5)
    x = synth.make_inputs(cfg, seed=80 + K)
    t = to_dev(x, cfg.dtype)
    O, Wf = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                              t["W_target"], cfg.eta, cfg.chunk, pad=pad)
    torch.cuda.synchronize()
    O, Wf = O.float().cpu().numpy(), Wf.cpu().numpy()
    O_ref, W_ref = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                                   x["W_target"], cfg.eta, cfg.chunk, pad=pad)
    W0 = np.broadcast_to(np.asarray(x["W_down0"], np.float64), W_ref.shape)
    e_o, e_dw = rel(O, O_ref), rel(Wf - W0, W_ref - W0)
    print(f"K={K} {pad}: O {e_o:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL, f"O error {e_o:.3e}"
    assert e_dw <= DW_TOL, f"dW error {e_dw:.3e}"


def test_continued_segment_with_64_taps(ttt):
    """A segment followed by 63 look-ahead rows (K = 64, sequence padding):
    the state it leaves equals the oracle's run over segment and rows."""
    K, T = 64, 512
    cfg = BASE.with_(name="taps64_continue", seq_len=T + K - 1, chunk=128, conv_k=K,
                     taps_std=float(K) ** -0.5)
    x = synth.make_inputs(cfg, seed=97)
    t = to_dev(x, cfg.dtype)
    W = t["W_down0"].float()[None].contiguous().clone()
    O = ttt.layer_forward_continue(t["H"][:, :T].contiguous(), t["X0"][:, :T].contiguous(),
                                   t["X0"][:, T:].contiguous(), t["Wg"], t["Wu"], W, t["taps"],
                                   t["W_target"], cfg.eta, cfg.chunk)
    torch.cuda.synchronize()
    O_ref, W_ref = ora.ttt_prefill(x["H"][:, :T], x["X0"], x["Wg"], x["Wu"], x["W_down0"],
                                   x["taps"], x["W_target"], cfg.eta, cfg.chunk)
    W0 = np.asarray(x["W_down0"], np.float64)
    e_o = rel(O.float().cpu().numpy(), O_ref)
    e_dw = rel(W.cpu().numpy() - W0, W_ref - W0)
    print(f"K=64 continued: O {e_o:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL and e_dw <= DW_TOL
