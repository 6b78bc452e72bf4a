"""CPU check of the segmented oracle evaluation that the full-size backward
parity test uses: segments chained through the state (forward) and the
state gradient (backward) give the oracle's one-piece result."""

import numpy as np

import oracle.ttt_oracle as ora
import synth
from test_parity_backward import GRADS, oracle_backward_segments, upstream


def test_segmented_oracle_is_the_oracle():
    """A small case with a ragged end, in four segments of two chunks."""
    cfg = synth.CONFIGS["tiny_amp"]
    x = synth.make_inputs(cfg, seq_len=200, seed=213)
    dO, dWf = upstream(x, cfg.dtype, seed=214)
    ref = ora.ttt_prefill_backward(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                                   x["W_target"], cfg.eta, 32, dO, dW_final=dWf)
    seg = oracle_backward_segments(x, dO, dWf, cfg.eta, 32, seg_chunks=2)
    for k in GRADS:
        np.testing.assert_allclose(seg[k], ref[k], rtol=1e-9, atol=1e-12, err_msg=k)


def test_segments_per_sequence_add_up():
    """Two sequences evaluated one at a time and combined (the per-token
    gradients side by side, the shared weights' gradients added) give the
    oracle's batch result."""
    cfg = synth.CONFIGS["tiny_amp"]
    x = synth.make_inputs(cfg, batch=2, seq_len=150, seed=9)
    dO, dWf = upstream(x, cfg.dtype, seed=10)
    one = ora.ttt_prefill_backward(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                                   x["W_target"], cfg.eta, 32, dO, dW_final=dWf)
    parts = []
    for b in range(2):
        xb = {k: (v[b:b + 1] if k in ("H", "X0") else v) for k, v in x.items()}
        parts.append(oracle_backward_segments(xb, dO[b:b + 1], dWf[b:b + 1], cfg.eta, 32,
                                              seg_chunks=2))
    for k in ("dH", "dX0"):
        np.testing.assert_allclose(np.concatenate([p[k] for p in parts]), one[k], rtol=1e-9,
                                   atol=1e-12, err_msg=k)
    for k in ("dWg", "dWu", "dtaps", "dW_target", "dW_down0"):
        np.testing.assert_allclose(parts[0][k] + parts[1][k], one[k], rtol=1e-9, atol=1e-12,
                                   err_msg=k)
