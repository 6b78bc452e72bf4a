"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances: max|err| / max|ref| <= 2e-2 for the bf16 output O and <= 1e-3
for the fp32 final state; the update itself, dW = W_final - W_down0, within
1e-2 of the reference update (the update is a few percent of W, so the raw
W check alone would hide a wrong update). The bf16 path rounds Z, V, the
state snapshots and O to bf16 (relative error 2^-9 each), which puts the
expected error near 4e-3 for O and 3e-3 for dW.

Sizes: the small configurations run the whole oracle. The full-size
configurations run exactly what the benchmark times, and are checked on
outputs the oracle can compute directly: rows of Z and V, every output of
the first chunks (the oracle runs those chunks with the conv's look-ahead
rows), and sampled entries of the final state.
"""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as ora
import synth

pytestmark = pytest.mark.gpu

O_TOL, W_TOL, DW_TOL, STEP_TOL = 2e-2, 1e-3, 1e-2, 1e-2


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import test_layer_gate_amd as m
    m.lib()
    return m


def rel(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(a - ref).max() / max(np.abs(ref).max(), 1e-30))


def to_dev(x, dtype):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(td) for k, v in x.items()}


def run_gpu(ttt, t, eta, chunk, **kw):
    O, Wf = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                              t["W_target"], eta, chunk, **kw)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), Wf.cpu().numpy()


def check_full(x, O, Wf, eta, chunk, pad="sequence", W0=None, raw_w=True):
    W0 = x["W_down0"] if W0 is None else W0
    O_ref, W_ref = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], W0, x["taps"],
                                   x["W_target"], eta, chunk, pad=pad)
    e_o = rel(O, O_ref)
    W0b = np.broadcast_to(np.asarray(W0, np.float64), W_ref.shape)
    e_dw = rel(Wf - W0b, W_ref - W0b)
    e_w = rel(Wf, W_ref)
    print(f"O {e_o:.2e}  W {e_w:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL, f"O error {e_o:.3e}"
    assert e_dw <= DW_TOL, f"dW error {e_dw:.3e}"
    if raw_w:
        assert e_w <= W_TOL, f"W error {e_w:.3e}"
    return e_o, e_w, e_dw


SMALL = ["tiny", "tiny_amp", "mid_amp"]


@pytest.mark.parametrize("name", SMALL)
def test_steps_match_oracle(ttt, name):
    cfg = synth.CONFIGS[name]
    x = synth.make_inputs(cfg)
    t = to_dev(x, cfg.dtype)
    Z = ttt.gated_activation(t["H"], t["Wg"], t["Wu"]).float().cpu().numpy()
    V = ttt.lm_target(t["X0"], t["taps"], t["W_target"], chunk=cfg.chunk).float().cpu().numpy()
    for b in range(cfg.batch):
        ez = rel(Z[b], ora.gated_activation(x["H"][b], x["Wg"], x["Wu"]))
        ev = rel(V[b], ora.lm_target(x["X0"][b], x["taps"], x["W_target"]))
        print(f"{name}: Z {ez:.2e} V {ev:.2e}")
        assert ez <= STEP_TOL and ev <= STEP_TOL


@pytest.mark.parametrize("schedule", ["prefix", "running"])
@pytest.mark.parametrize("pad", ["sequence", "chunk"])
@pytest.mark.parametrize("name", SMALL)
def test_forward_small(ttt, name, schedule, pad):
    cfg = synth.CONFIGS[name]
    x = synth.make_inputs(cfg)
    O, Wf = run_gpu(ttt, to_dev(x, cfg.dtype), cfg.eta, cfg.chunk, schedule=schedule, pad=pad)
    # Raw W check only where the update is small next to W (the amplified
    # configs make the update comparable to W on purpose).
    check_full(x, O, Wf, cfg.eta, cfg.chunk, pad=pad, raw_w=name == "tiny")


def test_ragged_batched_per_sequence_state(ttt):
    """B = 2, T = 1000 (not a multiple of the chunk, of 64 or of 256), each
    sequence with its own W_down0."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=2, seq_len=1000, seed=7)
    W0 = np.stack([x["W_down0"], synth.round_to_bf16(-0.5 * x["W_down0"])])
    t = to_dev(x, cfg.dtype)
    t["W_down0"] = torch.from_numpy(W0).to("cuda").to(torch.bfloat16)
    for schedule in ("prefix", "running"):
        O, Wf = run_gpu(ttt, t, cfg.eta, cfg.chunk, schedule=schedule)
        check_full(x, O, Wf, cfg.eta, cfg.chunk, W0=W0, raw_w=False)


@pytest.mark.parametrize("T,C", [(1, 64), (63, 64), (65, 64), (300, 128), (257, 256)])
def test_edge_lengths(ttt, T, C):
    cfg = synth.CONFIGS["tiny_amp"]
    x = synth.make_inputs(cfg, seq_len=T, seed=T)
    O, Wf = run_gpu(ttt, to_dev(x, cfg.dtype), cfg.eta, C)
    check_full(x, O, Wf, cfg.eta, C, raw_w=False)


def test_special_cases_reduce_to_plain_mlp(ttt):
    """eta = 0, zero taps, zero W_target: O is the plain gated MLP and the
    final state is W_down0 exactly."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg)
    t = to_dev(x, cfg.dtype)
    plain = ora.gated_activation(x["H"][0], x["Wg"], x["Wu"]) @ x["W_down0"].astype(np.float64).T
    for over in ({"eta": 0.0}, {"taps": torch.zeros_like(t["taps"])},
                 {"W_target": torch.zeros_like(t["W_target"])}):
        tt = dict(t)
        eta = over.pop("eta", cfg.eta)
        tt.update(over)
        O, Wf = run_gpu(ttt, tt, eta, cfg.chunk)
        assert rel(O[0], plain) <= O_TOL
        assert np.array_equal(Wf[0], x["W_down0"]), "final state must be W_down0 exactly"


def test_schedules_agree_bitwise(ttt):
    """Both schedules add the same 64-token products in the same order into
    an fp32 state, so their outputs are identical bit for bit."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, seq_len=1900, seed=3)
    t = to_dev(x, cfg.dtype)
    Op, Wp = run_gpu(ttt, t, cfg.eta, cfg.chunk, schedule="prefix")
    Or, Wr = run_gpu(ttt, t, cfg.eta, cfg.chunk, schedule="running")
    assert np.array_equal(Op, Or) and np.array_equal(Wp, Wr)


@pytest.mark.timeout(600)
def test_schedules_agree_bitwise_full_size(ttt):
    """The same at the Qwen3-4B 64k shape, where the running schedule's
    per-chunk apply uses 64-token tiles and the prefix schedule's 256-token
    ones: the tile width changes no sum."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    x = synth.make_inputs(cfg)
    t = to_dev(x, cfg.dtype)
    del x
    Op, Wp = run_gpu(ttt, t, cfg.eta, cfg.chunk, schedule="prefix")
    Or, Wr = run_gpu(ttt, t, cfg.eta, cfg.chunk, schedule="running")
    assert np.array_equal(Op, Or) and np.array_equal(Wp, Wr)


def test_deterministic(ttt):
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg)
    t = to_dev(x, cfg.dtype)
    a = run_gpu(ttt, t, cfg.eta, cfg.chunk)
    b = run_gpu(ttt, t, cfg.eta, cfg.chunk)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_chunk_causality(ttt):
    """Changing H in chunk j leaves every earlier chunk's output bitwise
    unchanged (apply uses the state from before the chunk's own update)."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg)
    t = to_dev(x, cfg.dtype)
    O, _ = run_gpu(ttt, t, cfg.eta, cfg.chunk)
    j, C = 3, cfg.chunk
    t2 = dict(t)
    t2["H"] = t["H"].clone()
    t2["H"][:, j * C:(j + 1) * C] += 1.0
    O2, _ = run_gpu(ttt, t2, cfg.eta, C)
    assert np.array_equal(O2[:, :j * C], O[:, :j * C])
    assert not np.array_equal(O2[:, (j + 1) * C:], O[:, (j + 1) * C:])


def test_error_writes_nothing(ttt):
    cfg = synth.CONFIGS["tiny_amp"]
    x = synth.make_inputs(cfg)
    t = to_dev(x, cfg.dtype)
    O = torch.full_like(t["H"], 7.0)
    Wf = torch.full((1, cfg.d_model, cfg.d_ff), 7.0, device="cuda")
    with pytest.raises(ttt.TTTError) as e:
        ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                          t["W_target"], cfg.eta, 100, out=O, W_down_final=Wf)
    assert e.value.name == "TTT_ERR_UNSUPPORTED"
    torch.cuda.synchronize()
    assert bool((O == 7.0).all()) and bool((Wf == 7.0).all())


def test_qwen3_4b_8k_full(ttt):
    """The Qwen3-4B-shaped 8k layer against the whole float64 recurrence."""
    cfg = synth.CONFIGS["qwen3_4b_8k"]
    x = synth.make_inputs(cfg)
    O, Wf = run_gpu(ttt, to_dev(x, cfg.dtype), cfg.eta, cfg.chunk)
    check_full(x, O, Wf, cfg.eta, cfg.chunk)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["qwen3_4b_64k", "llama31_8b_32k", "qwen3_14b_128k"])
def test_full_size_sampled(ttt, name):
    cfg = synth.CONFIGS[name]
    x = synth.make_inputs(cfg)
    C, K, eta = cfg.chunk, cfg.conv_k, cfg.eta
    t = to_dev(x, cfg.dtype)
    O, Wf = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                              t["W_target"], eta, C)
    n_chunks = 3 if name == "qwen3_4b_64k" else 2
    O_head = O[:, :n_chunks * C].float().cpu().numpy()
    rng = np.random.default_rng(1234)
    cs = np.unique(np.concatenate([[0, cfg.d_model - 1], rng.integers(0, cfg.d_model, 14)]))
    js = np.unique(np.concatenate([[0, cfg.d_ff - 1], rng.integers(0, cfg.d_ff, 14)]))
    W_s = Wf[:, cs][:, :, js].cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, C - 1, C, cfg.seq_len - 2, cfg.seq_len - 1],
                                     rng.integers(0, cfg.seq_len, 10)]))
    Z = ttt.gated_activation(t["H"], t["Wg"], t["Wu"])
    Z_s = Z[:, rows].float().cpu().numpy()
    del Z
    V = ttt.lm_target(t["X0"], t["taps"], t["W_target"], chunk=C)
    V_s = V[:, rows].float().cpu().numpy()
    del V, O, Wf, t
    torch.cuda.empty_cache()
    for b in range(cfg.batch):
        ez = rel(Z_s[b], ora.activation_rows(x["H"][b], x["Wg"], x["Wu"], rows))
        ev = rel(V_s[b], ora.target_rows(x["X0"][b], x["taps"], x["W_target"], rows))
        n = n_chunks * C
        O_ref, _ = ora.ttt_prefill(x["H"][b:b + 1, :n], x["X0"][b:b + 1, :n + K - 1], x["Wg"],
                                   x["Wu"], x["W_down0"], x["taps"], x["W_target"], eta, C)
        eo = rel(O_head[b], O_ref[0])
        W_ref = ora.final_state_entries(x["H"][b], x["X0"][b], x["Wg"], x["Wu"],
                                        x["W_down0"], x["taps"], x["W_target"], eta, cs, js)
        W0s = x["W_down0"][np.ix_(cs, js)].astype(np.float64)
        ew = rel(W_s[b], W_ref)
        edw = rel(W_s[b] - W0s, W_ref - W0s)
        print(f"{name}[{b}]: Z {ez:.2e} V {ev:.2e} O(first {n_chunks} chunks) {eo:.2e} "
              f"W {ew:.2e} dW {edw:.2e}", flush=True)
        assert ez <= STEP_TOL and ev <= STEP_TOL
        assert eo <= O_TOL and ew <= W_TOL and edw <= DW_TOL
