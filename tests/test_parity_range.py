"""GPU parity where the fp16 operand copies would leave fp16's range.

The update's operands Z^T and V^T, and the target's conv(X0) and
W_target^T, are fp16 copies (normal values from 2^-14 to 65504). Real
hidden states and learned projections are not bounded by Gaussian draws, so
these tests push each copy out of that range and check the layer against
the oracle (tolerances as in test_parity.py):

* |Z| near 1e5 (H drawn with std 100): Z^T would overflow;
* |conv(X0)| and |V| near 1e5 (X0 scaled by 2^16): both would overflow;
* W_target entries near 1e-7: W_target^T and V would flush to zero (with
  W_down0 = 0, so that the fp32 state can resolve so small an update).

Each producer notes its largest |value| and the copy is rewritten times a
power of two when that maximum is out of range, which the consumers divide
back out. Powers of two make this exact, which the scaling test checks bit
for bit: inputs that differ by a power of two, both out of range, give
results that differ by exactly that power.
"""

import numpy as np
import pytest
import torch

import oracle.ttt_oracle as ora
import synth
from test_parity import DW_TOL, O_TOL, W_TOL, rel, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import test_layer_gate_amd as m
    m.lib()
    return m


CFG = synth.CONFIGS["mid_amp"]       # T = 2048, C = 256, d = 256, f = 1024, K = 4


def case(kind, seed=70):
    x = synth.make_inputs(CFG, seed=seed)
    if kind == "big_z":
        x["H"] = synth.round_to_bf16(x["H"] * np.float32(100.0))
    elif kind == "big_y":
        x["X0"] = (x["X0"] * np.float32(2.0 ** 16)).astype(np.float32)
    elif kind == "tiny_wt":
        x["W_target"] = synth.round_to_bf16(x["W_target"] * np.float32(1.6e-6))
        # The whole update is then about 2e-7, far below the resolution an
        # fp32 state has next to |W_down0| up to 0.15 (its ulp is 1.5e-8, and
        # every 64-token step rounds at it): the state starts at zero, so that
        # it holds the update alone.
        x["W_down0"] = np.zeros_like(x["W_down0"])
    return x


def check(x, O, Wf, eta, chunk, what, pad="sequence", clip=None):
    O_ref, W_ref = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                                   x["W_target"], eta, chunk, pad=pad, clip=clip)
    W0 = np.broadcast_to(np.asarray(x["W_down0"], np.float64), W_ref.shape)
    e_o, e_w, e_dw = rel(O, O_ref), rel(Wf, W_ref), rel(Wf - W0, W_ref - W0)
    print(f"{what}: O {e_o:.2e}  W {e_w:.2e}  dW {e_dw:.2e}", flush=True)
    assert np.isfinite(O).all() and np.isfinite(Wf).all()
    assert e_o <= O_TOL and e_dw <= DW_TOL and e_w <= W_TOL


def test_the_cases_leave_fp16_range():
    """The inputs do what the test names say (on the oracle's values)."""
    x = case("big_z")
    Z = ora.gated_activation(x["H"][0], x["Wg"], x["Wu"])
    assert np.abs(Z).max() > 7e4
    x = case("big_y")
    Y = ora.conv_target_input(x["X0"][0], x["taps"])
    V = Y @ x["W_target"].astype(np.float64)
    assert np.abs(Y).max() > 7e4 and np.abs(V).max() * CFG.eta * 1024 > 7e4
    x = case("tiny_wt")
    wt = np.abs(x["W_target"])
    assert wt.max() < 1e-5 and np.median(wt) < 1e-6
    V = ora.lm_target(x["X0"][0], x["taps"], x["W_target"])
    assert np.abs(V).max() * CFG.eta * 1024 < 2.0 ** -14


@pytest.mark.parametrize("schedule", ["prefix", "running"])
@pytest.mark.parametrize("kind", ["big_z", "big_y", "tiny_wt"])
def test_out_of_range_matches_oracle(ttt, kind, schedule):
    x = case(kind)
    O, Wf = run_gpu(ttt, to_dev(x, "bf16"), CFG.eta, CFG.chunk, schedule=schedule)
    check(x, O, Wf, CFG.eta, CFG.chunk, f"{kind} {schedule}")


def test_out_of_range_clipped_and_packed(ttt):
    """Clipping's norms (taken from the rescaled V) and packed documents."""
    x = case("tiny_wt", seed=71)
    Z = ora.gated_activation(x["H"][0], x["Wg"], x["Wu"])
    V = ora.lm_target(x["X0"][0], x["taps"], x["W_target"])
    norms = [np.linalg.norm(CFG.eta * (V[a:a + CFG.chunk].T @ Z[a:a + CFG.chunk]))
             for a in range(0, CFG.seq_len, CFG.chunk)]
    clip = 0.5 * float(np.median(norms))
    t = to_dev(x, "bf16")
    O, Wf = run_gpu(ttt, t, CFG.eta, CFG.chunk, clip=clip)
    check(x, O, Wf, CFG.eta, CFG.chunk, "tiny_wt clipped", clip=clip)
    x = case("big_y", seed=72)
    starts = [0, 512, 1344]
    t = to_dev(x, "bf16")
    O, Wf = ttt.layer_forward_packed(t["H"][0], t["X0"][0], t["Wg"], t["Wu"], t["W_down0"],
                                     t["taps"], t["W_target"], CFG.eta, CFG.chunk, starts)
    torch.cuda.synchronize()
    O_ref, W_ref = ora.ttt_prefill_packed(x["H"][0], x["X0"][0], x["Wg"], x["Wu"],
                                          x["W_down0"], x["taps"], x["W_target"], CFG.eta,
                                          CFG.chunk, starts)
    e_o, e_w = rel(O.float().cpu().numpy(), O_ref), rel(Wf.cpu().numpy(), W_ref)
    print(f"big_y packed: O {e_o:.2e} W {e_w:.2e}", flush=True)
    assert e_o <= O_TOL and e_w <= W_TOL


def test_out_of_range_decode_and_target_step(ttt):
    """Decode (the chunk's Z^T rebuilt at the chunk's close) and the target
    step entry point (W_target^T and conv(X0) rescaled)."""
    x = case("big_z", seed=73)
    T, C = 768, CFG.chunk
    t = to_dev({k: (v[:, :T] if k in ("H", "X0") else v) for k, v in x.items()}, "bf16")
    W = t["W_down0"].float()[None].contiguous().clone()
    desc = ttt.make_desc(1, 1, CFG.d_model, CFG.d_ff, CFG.conv_k, 0, 0, 0, 1)
    ds = torch.empty(ttt.decode_state_size(desc, C), dtype=torch.uint8, device="cuda")
    ttt.decode_begin(W, C, ds, conv_k=CFG.conv_k)
    outs = [ttt.decode_step(t["H"][:, p], t["X0"][:, p], t["Wg"], t["Wu"], t["taps"],
                            t["W_target"], CFG.eta, C, p, W, ds) for p in range(T)]
    torch.cuda.synchronize()
    O = torch.stack(outs, 1).float().cpu().numpy()
    xs = {k: (v[:, :T] if k in ("H", "X0") else v) for k, v in x.items()}
    O_ref, W_ref, _ = ora.ttt_decode(xs["H"], xs["X0"], x["Wg"], x["Wu"], x["W_down0"],
                                     x["taps"], x["W_target"], CFG.eta, C)
    e_o, e_w = rel(O, O_ref), rel(W.cpu().numpy(), W_ref)
    print(f"big_z decode: O {e_o:.2e} W {e_w:.2e}", flush=True)
    assert e_o <= O_TOL and e_w <= W_TOL
    x = case("tiny_wt", seed=74)
    t = to_dev(x, "bf16")
    V = ttt.lm_target(t["X0"], t["taps"], t["W_target"], chunk=C).float().cpu().numpy()
    e_v = rel(V[0], ora.lm_target(x["X0"][0], x["taps"], x["W_target"]))
    print(f"tiny_wt target step: V {e_v:.2e}", flush=True)
    assert e_v <= 1e-2


def test_power_of_two_scaling_is_exact(ttt):
    """With W_down0 = 0, V and the final state are linear in X0 and O is too:
    X0 times 2^20 and times 2^26 (both far outside fp16's range for conv(X0)
    and V, so both are rescaled to the same fp16 values) give O and W_final
    that differ by exactly 2^6, bit for bit. The same for W_u times 2^14 and
    2^18 (Z scales by the factor, out of range in both; O by its square, the
    state by it)."""
    x = case("plain", seed=75)
    x["W_down0"] = np.zeros_like(x["W_down0"])
    def run(over):
        y = dict(x, **over)
        return run_gpu(ttt, to_dev(y, "bf16"), CFG.eta, CFG.chunk)
    O1, W1 = run({"X0": x["X0"] * np.float32(2.0 ** 20)})
    O2, W2 = run({"X0": x["X0"] * np.float32(2.0 ** 26)})
    assert np.isfinite(O1).all() and np.abs(W1).max() > 0
    assert np.array_equal(O1 * np.float32(2.0 ** 6), O2)
    assert np.array_equal(W1 * np.float32(2.0 ** 6), W2)
    O1, W1 = run({"Wu": x["Wu"] * np.float32(2.0 ** 14)})
    O2, W2 = run({"Wu": x["Wu"] * np.float32(2.0 ** 18)})
    assert np.array_equal(O1 * np.float32(2.0 ** 8), O2)
    assert np.array_equal(W1 * np.float32(2.0 ** 4), W2)
