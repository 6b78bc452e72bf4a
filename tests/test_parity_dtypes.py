"""GPU parity for the storage dtypes the ABI takes independently: the
activations H, X0 (and O) and the weights Wg, Wu, W_down0, taps, W_target
each bf16 or fp32. fp32 values here are not bf16-exact (drawn without
rounding), so the library's own rounding of fp32 inputs is exercised; the
oracle computes with the exact fp32 values. Prefill (both schedules), the
packed entry point and the decode step, against the CPU oracle; tolerances
as in test_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as ora
import synth
from test_parity import DW_TOL, O_TOL, rel

pytestmark = pytest.mark.gpu

ACTS = ("H", "X0")
WEIGHTS = ("Wg", "Wu", "W_down0", "taps", "W_target")
COMBOS = [("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")]


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import test_layer_gate_amd as m
    m.lib()
    return m


def inputs(act, wt, seed, seq_len=512):
    """mid_amp distributions; each group drawn exact in fp32, then rounded to
    bf16 where that group is stored in bf16 (so both sides see the same
    numbers for it)."""
    cfg = synth.CONFIGS["mid_amp"].with_(name="dtypes", dtype="f32", seq_len=seq_len,
                                         chunk=128)
    x = synth.make_inputs(cfg, seed=seed)
    dev = {}
    for k, v in x.items():
        bf = (act if k in ACTS else wt) == "bf16"
        if bf:
            x[k] = synth.round_to_bf16(v)
        t = torch.from_numpy(np.ascontiguousarray(x[k])).to("cuda")
        dev[k] = t.to(torch.bfloat16) if bf else t
    return cfg, x, dev


def check(O, Wf, O_ref, W_ref, W0, what):
    W0 = np.broadcast_to(np.asarray(W0, np.float64), W_ref.shape)
    e_o, e_dw = rel(O, O_ref), rel(Wf - W0, W_ref - W0)
    print(f"{what}: O {e_o:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL, f"O error {e_o:.3e}"
    assert e_dw <= DW_TOL, f"dW error {e_dw:.3e}"


@pytest.mark.parametrize("schedule", ["prefix", "running"])
@pytest.mark.parametrize("act,wt", COMBOS)
def test_prefill_dtypes(ttt, act, wt, schedule):
    cfg, x, t = inputs(act, wt, seed=61)
    O, Wf = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                              t["W_target"], cfg.eta, cfg.chunk, schedule=schedule)
    torch.cuda.synchronize()
    assert O.dtype == t["H"].dtype
    O_ref, W_ref = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                                   x["W_target"], cfg.eta, cfg.chunk)
    check(O.float().cpu().numpy(), Wf.cpu().numpy(), O_ref, W_ref, x["W_down0"],
          f"prefill act {act} weights {wt} {schedule}")


@pytest.mark.parametrize("act,wt", COMBOS)
def test_packed_dtypes(ttt, act, wt):
    cfg, x, t = inputs(act, wt, seed=62)
    starts = [0, 192, 256]
    O, Wf = ttt.layer_forward_packed(t["H"][0], t["X0"][0], t["Wg"], t["Wu"], t["W_down0"],
                                     t["taps"], t["W_target"], cfg.eta, cfg.chunk, starts)
    torch.cuda.synchronize()
    O_ref, W_ref = ora.ttt_prefill_packed(x["H"][0], x["X0"][0], x["Wg"], x["Wu"],
                                          x["W_down0"], x["taps"], x["W_target"], cfg.eta,
                                          cfg.chunk, starts)
    check(O.float().cpu().numpy(), Wf.cpu().numpy(), O_ref, W_ref, x["W_down0"],
          f"packed act {act} weights {wt}")


@pytest.mark.parametrize("act,wt", COMBOS)
def test_decode_dtypes(ttt, act, wt):
    cfg, x, t = inputs(act, wt, seed=63, seq_len=300)
    T, C = 300, cfg.chunk
    W = t["W_down0"].float()[None].contiguous().clone()
    desc = ttt.make_desc(1, 1, cfg.d_model, cfg.d_ff, cfg.conv_k,
                         1 if act == "f32" else 0, 1 if wt == "f32" else 0, 0,
                         ttt._binding.FLAG_PAD_CHUNK)
    ds = torch.empty(ttt.decode_state_size(desc, C), dtype=torch.uint8, device="cuda")
    ttt.decode_begin(W, C, ds, act_dtype=t["H"].dtype, weight_dtype=t["Wg"].dtype,
                     conv_k=cfg.conv_k)
    outs = []
    for pos in range(T):
        outs.append(ttt.decode_step(t["H"][:, pos].contiguous(), t["X0"][:, pos].contiguous(),
                                    t["Wg"], t["Wu"], t["taps"], t["W_target"], cfg.eta, C, pos,
                                    W, ds))
    torch.cuda.synchronize()
    O = torch.stack(outs, dim=1).float().cpu().numpy()
    O_ref, W_ref, pending = ora.ttt_decode(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"],
                                           x["taps"], x["W_target"], cfg.eta, C)
    assert pending == T % C
    check(O, W.cpu().numpy(), O_ref, W_ref, x["W_down0"], f"decode act {act} weights {wt}")
