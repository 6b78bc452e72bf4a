"""GPU parity of the prefill's backward pass (ttt_layer_backward) against
the oracle's ttt_prefill_backward, every gradient element by element.

The backward takes bf16 operands with fp32 accumulation and keeps every
chunk's state W_i and state gradient Gbar_{i+1} as bf16 copies, so each
gradient carries a few bf16 roundings of relative size 2^-9 along its chain
(the state, the activation factors, the operand copies): the bar is
max|err| / max|ref| <= 2e-2 per gradient, as for the forward's output.

The amplified configurations make the fast-weight term dominate the output,
so that a dropped or misplaced term of the chunk recurrence's reverse (the
eta V Gbar term of dZ, the state before rather than after a chunk, dW_final)
moves a gradient far past the bar.
"""

import numpy as np
import pytest
import torch

import oracle.ttt_oracle as ora
import synth
from test_parity import rel, to_dev

pytestmark = pytest.mark.gpu

BWD_TOL = 2e-2
GRADS = ("dH", "dX0", "dWg", "dWu", "dW_down0", "dtaps", "dW_target")


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import test_layer_gate_amd as m
    m.lib()
    return m


def upstream(x, dtype, seed, with_dwf=True):
    """dO [B, T, d] (exact in the activation dtype) and dW_final [B, d, f]
    fp32 (or None), both standard normal."""
    B, T, d = x["H"].shape
    f = x["Wg"].shape[0]
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal((B, T, d)).astype(np.float32)
    if dtype == "bf16":
        dO = synth.round_to_bf16(dO)
    dWf = rng.standard_normal((B, d, f)).astype(np.float32) if with_dwf else None
    return dO, dWf


def run_backward(ttt, x, dtype, eta, chunk, dO, dWf, pad="sequence", W0=None):
    t = to_dev(x, dtype)
    if W0 is not None:
        t["W_down0"] = torch.from_numpy(W0).to("cuda").to(t["Wg"].dtype)
    dO_t = torch.from_numpy(dO).to("cuda").to(t["H"].dtype)
    dWf_t = None if dWf is None else torch.from_numpy(dWf).to("cuda")
    g = ttt.layer_backward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                           t["W_target"], eta, chunk, dO_t, dW_final=dWf_t, pad=pad)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def check(x, g, eta, chunk, dO, dWf, what, pad="sequence", W0=None):
    W0 = x["W_down0"] if W0 is None else W0
    ref = ora.ttt_prefill_backward(x["H"], x["X0"], x["Wg"], x["Wu"], W0, x["taps"],
                                   x["W_target"], eta, chunk, dO, dW_final=dWf, pad=pad)
    errs = {k: rel(g[k], ref[k]) for k in GRADS}
    print(f"{what}: " + "  ".join(f"{k} {e:.2e}" for k, e in errs.items()), flush=True)
    for k in GRADS:
        assert g[k].shape == ref[k].shape, k
        assert np.isfinite(g[k]).all(), k
    bad = {k: e for k, e in errs.items() if not e <= BWD_TOL}
    assert not bad, f"{what}: {bad}"
    return errs


@pytest.mark.parametrize("pad", ["sequence", "chunk"])
@pytest.mark.parametrize("name", ["tiny_amp", "mid_amp"])
def test_backward_matches_oracle(ttt, name, pad):
    cfg = synth.CONFIGS[name]
    x = synth.make_inputs(cfg, seed=200)
    dO, dWf = upstream(x, cfg.dtype, seed=201)
    g = run_backward(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf, pad=pad)
    check(x, g, cfg.eta, cfg.chunk, dO, dWf, f"{name} {pad}", pad=pad)


def test_backward_fp32_operands(ttt):
    """fp32 activations and weights (the tiny configuration): cast to bf16
    inside, gradients still fp32."""
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg, seed=202)
    dO, dWf = upstream(x, cfg.dtype, seed=203)
    g = run_backward(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf)
    check(x, g, cfg.eta, cfg.chunk, dO, dWf, "tiny fp32")


@pytest.mark.parametrize("shared", [True, False])
def test_backward_ragged_batch(ttt, shared):
    """B = 2, T = 1000 (a partial last chunk and a partial 256-token tile);
    W_down0 shared (its gradient summed over the batch) or per sequence."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=2, seq_len=1000, seed=204)
    W0 = None if shared else np.stack([x["W_down0"], synth.round_to_bf16(-0.5 * x["W_down0"])])
    dO, dWf = upstream(x, cfg.dtype, seed=205)
    g = run_backward(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf, W0=W0)
    check(x, g, cfg.eta, cfg.chunk, dO, dWf, f"ragged B=2 shared={shared}", W0=W0)


def test_backward_without_state_gradient(ttt):
    """dW_final = NULL is a zero upstream gradient of the final state."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, seed=206)
    dO, _ = upstream(x, cfg.dtype, seed=207, with_dwf=False)
    g = run_backward(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, None)
    check(x, g, cfg.eta, cfg.chunk, dO, None, "dW_final none")


@pytest.mark.parametrize("T,C", [(1, 64), (65, 64), (300, 128), (257, 256)])
def test_backward_edge_lengths(ttt, T, C):
    cfg = synth.CONFIGS["tiny_amp"]
    x = synth.make_inputs(cfg, seq_len=T, seed=300 + T)
    dO, dWf = upstream(x, cfg.dtype, seed=400 + T)
    g = run_backward(ttt, x, cfg.dtype, cfg.eta, C, dO, dWf)
    check(x, g, cfg.eta, C, dO, dWf, f"T={T} C={C}")


def test_backward_state_gradient_only(ttt):
    """dO = 0: every gradient flows from dW_final through the updates alone
    (dZ = eta V Gbar, dV = eta Z Gbar^T with Gbar = dW_final in every
    chunk, and dW_down0 = dW_final exactly)."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, seed=208)
    dO, dWf = upstream(x, cfg.dtype, seed=209)
    dO = np.zeros_like(dO)
    g = run_backward(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf)
    check(x, g, cfg.eta, cfg.chunk, dO, dWf, "dO zero")
    assert np.array_equal(g["dW_down0"], dWf[0])


def test_backward_deterministic(ttt):
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=2, seq_len=700, seed=210)
    dO, dWf = upstream(x, cfg.dtype, seed=211)
    a = run_backward(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf)
    b = run_backward(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf)
    for k in GRADS:
        assert np.array_equal(a[k], b[k]), k


def oracle_backward_segments(x, dO, dWf, eta, chunk, seg_chunks=8):
    """The oracle's gradients of a long sequence (B = 1), in segments of
    seg_chunks chunks so that its memory stays bounded. The chain rule
    splits the backward exactly where the split/resume pin splits the
    forward: a segment [a, b) is the prefill from the state W_a with X0's
    K - 1 look-ahead rows, so its backward with dW_final = dL/dW_b returns
    the segment's gradients and dL/dW_a; the look-ahead rows' gradient
    belongs to the next segment's first rows."""
    T = x["H"].shape[1]
    K = x["taps"].shape[0]
    L = seg_chunks * chunk
    starts = list(range(0, T, L))
    # forward: the state at every segment start
    W = [np.asarray(x["W_down0"], np.float64)[None]]
    for a in starts[:-1]:
        b = min(a + L, T)
        _, Wb = ora.ttt_prefill(x["H"][:, a:b], x["X0"][:, a:min(b + K - 1, T)], x["Wg"],
                                x["Wu"], W[-1], x["taps"], x["W_target"], eta, chunk)
        W.append(Wb)
        print(f"  oracle forward to token {b}", flush=True)
    d, f = x["Wg"].shape[1], x["Wg"].shape[0]
    ref = {"dH": np.zeros(x["H"].shape), "dX0": np.zeros(x["X0"].shape),
           "dWg": np.zeros((f, d)), "dWu": np.zeros((f, d)), "dtaps": np.zeros((K, d)),
           "dW_target": np.zeros((d, d))}
    gbar = np.zeros((1, d, f)) if dWf is None else np.asarray(dWf, np.float64)
    for s in reversed(range(len(starts))):
        a = starts[s]
        b = min(a + L, T)
        e = min(b + K - 1, T)
        g = ora.ttt_prefill_backward(x["H"][:, a:b], x["X0"][:, a:e], x["Wg"], x["Wu"], W[s],
                                     x["taps"], x["W_target"], eta, chunk, dO[:, a:b],
                                     dW_final=gbar)
        ref["dH"][:, a:b] = g["dH"]
        ref["dX0"][:, a:e] += g["dX0"]
        for k in ("dWg", "dWu", "dtaps", "dW_target"):
            ref[k] += g[k]
        gbar = g["dW_down0"]
        print(f"  oracle backward from token {b}", flush=True)
    ref["dW_down0"] = gbar[0]
    return ref


def test_backward_full_size_whole_sequence(ttt):
    """The Qwen3-4B shape at T = 65536 (the benchmark's backward call): every
    gradient over the whole sequence against the segmented oracle."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    x = synth.make_inputs(cfg)
    dO, dWf = upstream(x, cfg.dtype, seed=212)
    g = run_backward(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf)
    print("  GPU backward done", flush=True)
    ref = oracle_backward_segments(x, dO, dWf, cfg.eta, cfg.chunk)
    errs = {k: rel(g[k], ref[k]) for k in GRADS}
    print("qwen3_4b_64k: " + "  ".join(f"{k} {e:.2e}" for k, e in errs.items()), flush=True)
    for k in GRADS:
        assert np.isfinite(g[k]).all(), k
    bad = {k: e for k, e in errs.items() if not e <= BWD_TOL}
    assert not bad, bad



# ---- training: ttt_layer_forward_train, then ttt_layer_backward_saved ----

def run_train(ttt, x, dtype, eta, chunk, dO, dWf, pad="sequence", W0=None):
    t = to_dev(x, dtype)
    if W0 is not None:
        t["W_down0"] = torch.from_numpy(W0).to("cuda").to(t["Wg"].dtype)
    O, Wf, saved = ttt.layer_forward_train(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"],
                                           t["taps"], t["W_target"], eta, chunk, pad=pad)
    dO_t = torch.from_numpy(dO).to("cuda").to(t["H"].dtype)
    dWf_t = None if dWf is None else torch.from_numpy(dWf).to("cuda")
    g = ttt.layer_backward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                           t["W_target"], eta, chunk, dO_t, dW_final=dWf_t, pad=pad, saved=saved)
    O2, Wf2 = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                                t["W_target"], eta, chunk, pad=pad, schedule="prefix")
    torch.cuda.synchronize()
    # the training forward's outputs are the prefill's, bit for bit
    assert torch.equal(O, O2) and torch.equal(Wf, Wf2)
    return {k: v.cpu().numpy() for k, v in g.items()}


@pytest.mark.parametrize("pad", ["sequence", "chunk"])
@pytest.mark.parametrize("name", ["tiny_amp", "mid_amp"])
def test_saved_backward_matches_oracle(ttt, name, pad):
    cfg = synth.CONFIGS[name]
    x = synth.make_inputs(cfg, seed=220)
    dO, dWf = upstream(x, cfg.dtype, seed=221)
    g = run_train(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf, pad=pad)
    check(x, g, cfg.eta, cfg.chunk, dO, dWf, f"saved {name} {pad}", pad=pad)


@pytest.mark.parametrize("shared", [True, False])
def test_saved_backward_ragged_batch(ttt, shared):
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=2, seq_len=1000, seed=222)
    W0 = None if shared else np.stack([x["W_down0"], synth.round_to_bf16(-0.5 * x["W_down0"])])
    dO, dWf = upstream(x, cfg.dtype, seed=223)
    g = run_train(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf, W0=W0)
    check(x, g, cfg.eta, cfg.chunk, dO, dWf, f"saved ragged B=2 shared={shared}", W0=W0)


def test_saved_backward_fp32_and_no_state_gradient(ttt):
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg, seed=224)
    dO, _ = upstream(x, cfg.dtype, seed=225, with_dwf=False)
    g = run_train(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, None)
    check(x, g, cfg.eta, cfg.chunk, dO, None, "saved tiny fp32, dW_final none")


def test_saved_backward_full_size_whole_sequence(ttt):
    """The training step at the Qwen3-4B shape, T = 65536: the saved
    backward's gradients over the whole sequence against the segmented
    oracle."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    x = synth.make_inputs(cfg)
    dO, dWf = upstream(x, cfg.dtype, seed=226)
    g = run_train(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf)
    print("  GPU training step done", flush=True)
    ref = oracle_backward_segments(x, dO, dWf, cfg.eta, cfg.chunk)
    errs = {k: rel(g[k], ref[k]) for k in GRADS}
    print("saved qwen3_4b_64k: " + "  ".join(f"{k} {e:.2e}" for k, e in errs.items()), flush=True)
    for k in GRADS:
        assert np.isfinite(g[k]).all(), k
    bad = {k: e for k, e in errs.items() if not e <= BWD_TOL}
    assert not bad, bad


def test_backward_full_size_two_sequences(ttt):
    """The LLaMA-3.1-8B shape (B = 2, T = 32768, d 4096, d_ff 14336, one
    shared W_down0): every gradient over both whole sequences against the
    segmented oracle, run per sequence (the sequences share only W_down0,
    W_g, W_u, the taps and W_target, whose gradients add up)."""
    cfg = synth.CONFIGS["llama31_8b_32k"]
    x = synth.make_inputs(cfg)
    dO, dWf = upstream(x, cfg.dtype, seed=227)
    g = run_backward(ttt, x, cfg.dtype, cfg.eta, cfg.chunk, dO, dWf)
    print("  GPU backward done", flush=True)
    ref = None
    for b in range(cfg.batch):
        xb = {k: (v[b:b + 1] if k in ("H", "X0") else v) for k, v in x.items()}
        rb = oracle_backward_segments(xb, dO[b:b + 1], dWf[b:b + 1], cfg.eta, cfg.chunk)
        if ref is None:
            ref = {k: (np.zeros((cfg.batch,) + v.shape[1:]) if k in ("dH", "dX0") else v)
                   for k, v in rb.items()}
        else:
            for k in ("dWg", "dWu", "dtaps", "dW_target", "dW_down0"):
                ref[k] = ref[k] + rb[k]
        ref["dH"][b] = rb["dH"][0]
        ref["dX0"][b] = rb["dX0"][0]
        print(f"  oracle sequence {b} done", flush=True)
    errs = {k: rel(g[k], ref[k]) for k in GRADS}
    print("llama31_8b_32k: " + "  ".join(f"{k} {e:.2e}" for k, e in errs.items()), flush=True)
    for k in GRADS:
        assert g[k].shape == ref[k].shape, k
        assert np.isfinite(g[k]).all(), k
    bad = {k: e for k, e in errs.items() if not e <= BWD_TOL}
    assert not bad, bad


def test_backward_eta_zero(ttt):
    """eta = 0: the layer is the plain gated MLP (O = Z W_down0^T), so no
    gradient reaches the target path (dX0, dtaps and dW_target exactly
    zero) and the rest matches the oracle."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, seed=228)
    dO, dWf = upstream(x, cfg.dtype, seed=229)
    g = run_backward(ttt, x, cfg.dtype, 0.0, cfg.chunk, dO, dWf)
    for k in ("dX0", "dtaps", "dW_target"):
        assert not np.any(g[k]), k
    check(x, g, 0.0, cfg.chunk, dO, dWf, "eta 0")
