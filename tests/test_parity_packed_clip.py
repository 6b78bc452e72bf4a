"""GPU parity for packed documents with update-norm clipping
(ttt_layer_forward_packed_clipped) against the oracle's ttt_prefill_packed
with a limit: the state returns to W_down0 at every document start, and each
chunk's update eta V_i^T Z_i, with chunks counted from the document's start,
is scaled by min(1, clip / ||eta V_i^T Z_i||_F) (iplexlaw explainer §6). The
limit is a fraction of the median of the chunks' update norms: 0.9 or 0.95
of it (most chunks clipped, some not; no norm at the limit itself) or 0.3
of it (all clipped hard). Tolerances as in test_parity.py; clipping must
move the update by at least five times the GPU's error, so that the check
tells a clipped update from an unclipped one."""
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


def doc_chunk_norms(x, eta, C, starts):
    """eta * ||V_i^T Z_i||_F of every chunk of every document, each document
    on its own tokens (its conv stops at its end)."""
    T = x["H"].shape[1]
    bounds = list(starts) + [T]
    out = []
    for a, e in zip(bounds, bounds[1:]):
        Z = ora.gated_activation(x["H"][0, a:e], x["Wg"], x["Wu"])
        V = ora.lm_target(x["X0"][0, a:e], x["taps"], x["W_target"])
        out += [float(np.linalg.norm(eta * (V[c:c + C].T @ Z[c:c + C])))
                for c in range(0, e - a, C)]
    return out


def run_gpu(ttt, x, dtype, eta, C, starts, clip, **kw):
    t = to_dev(x, dtype)
    O, Wf = ttt.layer_forward_packed(t["H"][0], t["X0"][0], t["Wg"], t["Wu"], t["W_down0"],
                                     t["taps"], t["W_target"], eta, C, starts, clip=clip, **kw)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), Wf.cpu().numpy()


def check(x, O, Wf, eta, C, starts, clip, pad="sequence"):
    args = (x["H"][0], x["X0"][0], x["Wg"], x["Wu"], x["W_down0"], x["taps"], x["W_target"],
            eta, C, starts)
    O_ref, W_ref = ora.ttt_prefill_packed(*args, pad=pad, clip=clip)
    _, W_free = ora.ttt_prefill_packed(*args, pad=pad)
    W0 = np.asarray(x["W_down0"], np.float64)
    e_o, e_dw = rel(O, O_ref), rel(Wf - W0, W_ref - W0)
    gap = rel(W_free - W0, W_ref - W0)
    print(f"docs {starts} clip {clip:.3e}: O {e_o:.2e}  dW {e_dw:.2e}  "
          f"(clipping moves dW by {gap:.2e})", flush=True)
    assert e_o <= O_TOL, f"O error {e_o:.3e}"
    assert e_dw <= DW_TOL, f"dW error {e_dw:.3e}"
    assert gap >= 5 * e_dw, "the check cannot tell the clipped update from the unclipped one"


# 2 chunks, 64 tokens, 3 chunks, 2.75 chunks (chunk 256)
MIXED = [0, 512, 576, 1344]


@pytest.mark.parametrize("strength", [0.9, 0.3])
@pytest.mark.parametrize("schedule", ["prefix", "running"])
def test_packed_clipped_matches_oracle(ttt, schedule, strength):
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=1, seed=55)
    clip = strength * float(np.median(doc_chunk_norms(x, cfg.eta, cfg.chunk, MIXED)))
    O, Wf = run_gpu(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, MIXED, clip, schedule=schedule)
    check(x, O, Wf, cfg.eta, cfg.chunk, MIXED, clip)


def test_packed_clipped_chunk_padding_ragged(ttt):
    """Chunk-local conv padding, T = 1000 (the last document ragged: chunks
    of 512 and 168 tokens), chunks of 512 tokens, so that a chunk's norm sums
    several 256-token Gram blocks, some of them past a short chunk's end."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=1, seq_len=1000, seed=56)
    starts, C = [0, 320], 512
    clip = 0.95 * float(np.median(doc_chunk_norms(x, cfg.eta, C, starts)))
    O, Wf = run_gpu(ttt, x, cfg.dtype, cfg.eta, C, starts, clip, pad="chunk")
    check(x, O, Wf, cfg.eta, C, starts, clip, pad="chunk")


def test_packed_loose_clip_is_packed(ttt):
    """A limit above every chunk's norm gives ttt_layer_forward_packed bit
    for bit."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=1, seed=57)
    O1, W1 = run_gpu(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, MIXED, 1e30)
    O2, W2 = run_gpu(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, MIXED, None)
    assert np.array_equal(O1, O2) and np.array_equal(W1, W2)


def test_packed_clipped_qwen_widths(ttt):
    """The Qwen3-4B widths (d_model 2560, d_ff 9728; the packed update's
    mixed wide and narrow tiles) with three documents and chunk 256."""
    cfg = synth.CONFIGS["mid_amp"].with_(name="packed_clip_qwen", seq_len=768, d_model=2560,
                                         d_ff=9728)
    x = synth.make_inputs(cfg, batch=1, seed=58)
    starts, C = [0, 320, 448], 256
    clip = 0.95 * float(np.median(doc_chunk_norms(x, cfg.eta, C, starts)))
    O, Wf = run_gpu(ttt, x, cfg.dtype, cfg.eta, C, starts, clip)
    check(x, O, Wf, cfg.eta, C, starts, clip)
