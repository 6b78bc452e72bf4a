"""GPU parity for continued documents (ttt_layer_forward_continue): a
document prefilled in segments, each segment starting from the fp32 state
the previous one returned and reading the next segment's first K - 1 X0
rows through the conv (iplexlaw explainer §6, §8: the fast weight keeps
changing over the whole document). Checked against the CPU oracle's single
run over the whole document, against the oracle run of one segment from the
GPU's own state, and against the one-call GPU result. Tolerances as in
test_parity.py."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as ora
import synth
from test_parity import DW_TOL, O_TOL, W_TOL, rel, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import test_layer_gate_amd as m
    m.lib()
    return m


def state_of(W0, B):
    """The first segment's state: W_down0 widened to fp32, one per sequence."""
    W = W0.float()
    return (W.expand(B, *W.shape) if W.dim() == 2 else W).contiguous().clone()


def run_segments(ttt, t, eta, chunk, cuts, K, W_state=None, lookahead=True, **kw):
    """Runs the sequence as segments [cuts[i], cuts[i+1]) (cuts from 0 to T),
    each continuing the state; returns O [B, T, d] (fp32, host) and the state."""
    B = t["H"].shape[0]
    W = state_of(t["W_down0"], B) if W_state is None else W_state
    outs = []
    for a, e in zip(cuts[:-1], cuts[1:]):
        nxt = t["X0"][:, e:e + K - 1].contiguous() if lookahead and e < cuts[-1] else None
        if nxt is not None and nxt.shape[1] == 0:
            nxt = None
        O = ttt.layer_forward_continue(t["H"][:, a:e].contiguous(),
                                       t["X0"][:, a:e].contiguous(), nxt, t["Wg"], t["Wu"],
                                       W, t["taps"], t["W_target"], eta, chunk, **kw)
        outs.append(O)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1).float().cpu().numpy(), W.cpu().numpy()


def check(x, O, Wf, eta, chunk, pad="sequence", raw_w=True, what=""):
    O_ref, W_ref = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"],
                                   x["taps"], x["W_target"], eta, chunk, pad=pad)
    W0 = np.broadcast_to(np.asarray(x["W_down0"], np.float64), W_ref.shape)
    e_o, e_w, e_dw = rel(O, O_ref), rel(Wf, W_ref), rel(Wf - W0, W_ref - W0)
    print(f"{what}: O {e_o:.2e}  W {e_w:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL, f"O error {e_o:.3e}"
    assert e_dw <= DW_TOL, f"dW error {e_dw:.3e}"
    if raw_w:
        assert e_w <= W_TOL, f"W error {e_w:.3e}"


CASES = {
    # name: (config, overrides, segment cuts inside [0, T])
    "mid_amp_halves": ("mid_amp", {}, [1024]),
    "mid_amp_three": ("mid_amp", {}, [256, 1280]),
    "mid_amp_b2_ragged": ("mid_amp", dict(batch=2, seq_len=1000, seed=5), [512]),
    "tiny_f32": ("tiny", {}, [64, 192]),
}


@pytest.mark.parametrize("schedule", ["prefix", "running"])
@pytest.mark.parametrize("pad", ["sequence", "chunk"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_segments_match_one_oracle_run(ttt, case, pad, schedule):
    name, over, cuts = CASES[case]
    cfg = synth.CONFIGS[name]
    x = synth.make_inputs(cfg, **over)
    T = x["H"].shape[1]
    t = to_dev(x, cfg.dtype)
    O, Wf = run_segments(ttt, t, cfg.eta, cfg.chunk, [0] + cuts + [T], cfg.conv_k,
                         schedule=schedule, pad=pad)
    check(x, O, Wf, cfg.eta, cfg.chunk, pad=pad, what=case)


def test_segment_from_the_gpu_state(ttt):
    """The second segment alone against the oracle started from the state
    the GPU returned for the first: the fp32 state input and its in-place
    update, with the second segment ragged (T = 1000, C = 256)."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=2, seq_len=1000, seed=6)
    t = to_dev(x, cfg.dtype)
    _, W1 = run_segments(ttt, t, cfg.eta, cfg.chunk, [0, 512], cfg.conv_k)
    W = torch.from_numpy(W1).to("cuda")
    H2, X2 = t["H"][:, 512:].contiguous(), t["X0"][:, 512:].contiguous()
    O2 = ttt.layer_forward_continue(H2, X2, None, t["Wg"], t["Wu"], W, t["taps"],
                                    t["W_target"], cfg.eta, cfg.chunk)
    torch.cuda.synchronize()
    O_ref, W_ref = ora.ttt_prefill(x["H"][:, 512:], x["X0"][:, 512:], x["Wg"], x["Wu"], W1,
                                   x["taps"], x["W_target"], cfg.eta, cfg.chunk)
    e_o = rel(O2.float().cpu().numpy(), O_ref)
    e_dw = rel(W.cpu().numpy() - W1, W_ref - W1)
    print(f"second segment: O {e_o:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL and e_dw <= DW_TOL


@pytest.mark.parametrize("n_next", [0, 1, 2, 3])
def test_partial_lookahead(ttt, n_next):
    """Fewer look-ahead rows than K - 1: rows past them read as zero."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, seed=8)
    T = 768
    t = to_dev(x, cfg.dtype)
    W = state_of(t["W_down0"], 1)
    nxt = t["X0"][:, T:T + n_next].contiguous() if n_next else None
    O = ttt.layer_forward_continue(t["H"][:, :T].contiguous(), t["X0"][:, :T].contiguous(),
                                   nxt, t["Wg"], t["Wu"], W, t["taps"], t["W_target"],
                                   cfg.eta, cfg.chunk)
    torch.cuda.synchronize()
    O_ref, W_ref = ora.ttt_prefill(x["H"][:, :T], x["X0"][:, :T + n_next], x["Wg"], x["Wu"],
                                   x["W_down0"], x["taps"], x["W_target"], cfg.eta, cfg.chunk)
    W0 = np.asarray(x["W_down0"], np.float64)
    e_o = rel(O.float().cpu().numpy(), O_ref)
    e_dw = rel(W.cpu().numpy() - W0, W_ref - W0)
    print(f"n_next={n_next}: O {e_o:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL and e_dw <= DW_TOL


@pytest.mark.parametrize("schedule", ["prefix", "running"])
def test_split_is_the_one_call_result(ttt, schedule):
    """Split at 1024 tokens (a multiple of the chunk and of the kernels'
    tile groups), two calls run the one call's arithmetic in the same order:
    O and the final state are bit-identical to ttt_layer_forward's."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, seed=12)
    t = to_dev(x, cfg.dtype)
    O, Wf = run_segments(ttt, t, cfg.eta, cfg.chunk, [0, 1024, 2048], cfg.conv_k,
                         schedule=schedule)
    O1, W1 = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                               t["W_target"], cfg.eta, cfg.chunk, schedule=schedule)
    torch.cuda.synchronize()
    assert np.array_equal(O, O1.float().cpu().numpy())
    assert np.array_equal(Wf, W1.cpu().numpy())


def test_lookahead_rows_are_read_only_with_sequence_padding(ttt):
    """With sequence padding the look-ahead rows change the state (the last
    tokens' targets read them); with chunk padding they are never read."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, seed=13)
    t = to_dev(x, cfg.dtype)
    res = {}
    for pad in ("sequence", "chunk"):
        for la in (True, False):
            _, res[pad, la] = run_segments(ttt, t, cfg.eta, cfg.chunk, [0, 1024, 2048],
                                           cfg.conv_k, lookahead=la, pad=pad)
    assert not np.array_equal(res["sequence", True], res["sequence", False])
    assert np.array_equal(res["chunk", True], res["chunk", False])


@pytest.mark.timeout(900)
def test_continue_full_size_sampled(ttt):
    """Qwen3-4B shape, a 64k-token segment continuing a document: the state
    comes in as fp32 (W_down0 plus a perturbation no bf16 value carries) and
    three look-ahead rows follow. Checked on the first chunk's outputs (the
    incoming state applied) and on sampled entries of the final state, which
    depend on the look-ahead rows through the last tokens' targets."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    x = synth.make_inputs(cfg, seq_len=cfg.seq_len + cfg.conv_k - 1)
    T, C, K, eta = cfg.seq_len, cfg.chunk, cfg.conv_k, cfg.eta
    rng = np.random.default_rng(21)
    W_in = (x["W_down0"].astype(np.float32)
            + rng.standard_normal(x["W_down0"].shape).astype(np.float32) * 1e-3)[None]
    t = to_dev({k: v for k, v in x.items() if k not in ("H", "X0")}, cfg.dtype)
    H = torch.from_numpy(x["H"][:, :T]).to("cuda").to(torch.bfloat16)
    X0 = torch.from_numpy(x["X0"][:, :T]).to("cuda").to(torch.bfloat16)
    nxt = torch.from_numpy(x["X0"][:, T:]).to("cuda").to(torch.bfloat16).contiguous()
    W = torch.from_numpy(W_in).to("cuda")
    O = ttt.layer_forward_continue(H, X0, nxt, t["Wg"], t["Wu"], W, t["taps"],
                                   t["W_target"], eta, C)
    torch.cuda.synchronize()
    O0 = O[0, :C].float().cpu().numpy()
    Wf = W[0].cpu().numpy()
    del H, X0, O, W, t
    torch.cuda.empty_cache()
    O_ref = ora.activation_rows(x["H"][0], x["Wg"], x["Wu"], np.arange(C)) @ \
        W_in[0].astype(np.float64).T
    eo = rel(O0, O_ref)
    cs = np.unique(np.concatenate([[0, cfg.d_model - 1], rng.integers(0, cfg.d_model, 14)]))
    js = np.unique(np.concatenate([[0, cfg.d_ff - 1], rng.integers(0, cfg.d_ff, 14)]))
    W_ref = ora.final_state_entries(x["H"][0, :T], x["X0"][0], x["Wg"], x["Wu"], W_in[0],
                                    x["taps"], x["W_target"], eta, cs, js)
    W0s = W_in[0][np.ix_(cs, js)].astype(np.float64)
    W_s = Wf[np.ix_(cs, js)]
    ew, edw = rel(W_s, W_ref), rel(W_s - W0s, W_ref - W0s)
    print(f"first chunk O {eo:.2e}; final state W {ew:.2e} dW {edw:.2e}", flush=True)
    assert eo <= O_TOL and ew <= W_TOL and edw <= DW_TOL
