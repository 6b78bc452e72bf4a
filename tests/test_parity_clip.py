"""GPU parity for update-norm clipping (ttt_layer_forward_clipped) against
the oracle's clipped recurrence: every chunk's update eta V_i^T Z_i scaled by
min(1, clip / ||eta V_i^T Z_i||_F) (iplexlaw explainer §6). The limit is
set to the median of the chunks' update norms, so about half of the chunks
are clipped and half are not, or to 0.3 times it, so that nearly all are
clipped hard. Tolerances as in test_parity.py; in addition, clipping must
move the update by at least five times the GPU's error against the clipped
reference, so that the check tells a clipped update from an unclipped one."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as ora
import synth
from test_parity import DW_TOL, O_TOL, check_whole_sequence, rel, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import test_layer_gate_amd as m
    m.lib()
    return m


def chunk_update_norms(x, eta, C, b=0):
    Z = ora.gated_activation(x["H"][b], x["Wg"], x["Wu"])
    V = ora.lm_target(x["X0"][b], x["taps"], x["W_target"])
    T = Z.shape[0]
    return [float(np.linalg.norm(eta * (V[a:a + C].T @ Z[a:a + C]))) for a in range(0, T, C)]


def run_clip(ttt, x, dtype, eta, C, clip, **kw):
    t = to_dev(x, dtype)
    O, Wf = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                              t["W_target"], eta, C, clip=clip, **kw)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), Wf.cpu().numpy()


def check_clip(x, O, Wf, eta, C, clip, pad="sequence"):
    O_ref, W_ref = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                                   x["W_target"], eta, C, pad=pad, clip=clip)
    W0 = np.broadcast_to(np.asarray(x["W_down0"], np.float64), W_ref.shape)
    e_o, e_dw = rel(O, O_ref), rel(Wf - W0, W_ref - W0)
    _, W_free = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                                x["W_target"], eta, C, pad=pad)
    gap = rel(W_free - W0, W_ref - W0)     # how far clipping moves the update
    print(f"clip {clip:.3e}: O {e_o:.2e}  dW {e_dw:.2e}  (clipping moves dW by {gap:.2e})",
          flush=True)
    assert e_o <= O_TOL and e_dw <= DW_TOL
    assert gap >= 5 * e_dw, "the check cannot tell the clipped update from the unclipped one"


@pytest.mark.parametrize("strength", [1.0, 0.3])
@pytest.mark.parametrize("schedule", ["prefix", "running"])
@pytest.mark.parametrize("name,T", [("mid_amp", 2048), ("mid_amp", 1000), ("tiny_amp", 256)])
def test_clipped_matches_oracle(ttt, name, T, schedule, strength):
    cfg = synth.CONFIGS[name]
    x = synth.make_inputs(cfg, seq_len=T, seed=40 + T)
    clip = strength * float(np.median(chunk_update_norms(x, cfg.eta, cfg.chunk)))
    O, Wf = run_clip(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, clip, schedule=schedule)
    check_clip(x, O, Wf, cfg.eta, cfg.chunk, clip)


def test_loose_clip_is_the_plain_layer(ttt):
    """A limit above every chunk's norm leaves all scales at 1: the result is
    bit-identical to ttt_layer_forward."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg)
    t = to_dev(x, cfg.dtype)
    O1, W1 = run_clip(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, 1e30)
    O2, W2 = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                               t["W_target"], cfg.eta, cfg.chunk)
    torch.cuda.synchronize()
    assert np.array_equal(O1, O2.float().cpu().numpy())
    assert np.array_equal(W1, W2.cpu().numpy())


@pytest.mark.timeout(900)
def test_clip_full_size_whole_sequence(ttt):
    """Qwen3-4B shape at 64k tokens with a limit of half the first chunk's
    update norm (so it clips): every output of every chunk and every entry
    of the final state against the oracle's clipped run over the whole
    sequence (in segments). eta is 10x the config's, so that the fast-weight
    term (about 3% of O at the config's eta) is large enough for the check
    to tell clipped from unclipped, which the first three chunks' unclipped
    oracle run confirms. A limit above every update norm gives the
    unclipped layer bit for bit."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    x = synth.make_inputs(cfg)
    C, eta, K, n = cfg.chunk, 10 * cfg.eta, cfg.conv_k, 3 * cfg.chunk
    head = {k: (v[:, :n + K - 1] if k == "X0" else v[:, :n] if k == "H" else v)
            for k, v in x.items()}
    norms = chunk_update_norms(dict(head, X0=x["X0"][:, :n]), eta, C)
    clip = 0.5 * norms[0]
    O, Wf = run_clip(ttt, x, cfg.dtype, eta, C, clip)
    O_ref, _ = ora.ttt_prefill(head["H"], head["X0"], x["Wg"], x["Wu"], x["W_down0"],
                               x["taps"], x["W_target"], eta, C, clip=clip)
    O_free, _ = ora.ttt_prefill(head["H"], head["X0"], x["Wg"], x["Wu"], x["W_down0"],
                                x["taps"], x["W_target"], eta, C)
    gap = rel(O_free[:, 2 * C:n], O_ref[:, 2 * C:n])
    e3 = rel(O[:, 2 * C:n], O_ref[:, 2 * C:n])
    print(f"64k clipped: third chunk {e3:.2e} (clipping moves it by {gap:.2e})", flush=True)
    assert e3 <= O_TOL
    assert gap >= 5 * e3, "the check cannot tell the clipped outputs from the unclipped ones"
    check_whole_sequence(x, O, Wf, eta, C, "qwen3_4b_64k clipped", clip=clip)
    O_loose, W_loose = run_clip(ttt, x, cfg.dtype, eta, C, 1e30)
    O_plain, W_plain = run_clip(ttt, x, cfg.dtype, eta, C, None)
    assert np.array_equal(O_loose, O_plain) and np.array_equal(W_loose, W_plain)
