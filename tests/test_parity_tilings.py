"""GPU parity for the update's tile layouts. The update covers the state in
256 x 256 regions and runs whole rounds of wide 256 x 256 tiles, one per
compute unit, plus (when the regions left over fill at most half a round)
two narrow 256 x 128 tiles per leftover region. These shapes put the
boundary between the two kinds of tiles inside a sequence of a batch, at a
batch edge, leave a narrow half wholly past d_model, and run one round of
wide tiles only; each is checked against the CPU oracle (amplified
distributions, so that the update is a large part of the output; tolerances
as in test_parity.py). The region counts below assume 256 compute units;
on another part the same shapes still run, split differently.
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
CASES = {
    # name: (batch, seq_len, chunk, d_model, d_ff); regions = B * ceil(d/256) * ceil(f/256)
    # 4 x 3 x 32 = 384: 256 wide, then 128 regions as narrow pairs; the
    # boundary falls inside the third sequence.
    "boundary_in_sequence": (4, 256, 128, 768, 8192),
    # 2 x 6 x 22 = 264: 256 wide, 8 regions narrow, inside the second sequence.
    "few_narrow": (2, 256, 128, 1536, 5632),
    # 1 x 5 x 32 = 160 (more than half a round): one round of wide tiles.
    "wide_only": (1, 256, 128, 1280, 8192),
    # 1 x 3 x 5 = 15: narrow tiles only; d_model = 640 leaves the second half
    # of the last region column past d_model, and d_ff = 1088 a last region
    # row with 64 valid rows.
    "narrow_partial": (1, 320, 128, 640, 1088),
}


@pytest.mark.parametrize("schedule", ["prefix", "running"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_update_tilings_match_oracle(ttt, case, schedule):
    B, T, C, d, f = CASES[case]
    cfg = BASE.with_(name=case, batch=B, seq_len=T, chunk=C, d_model=d, d_ff=f)
    x = synth.make_inputs(cfg, seed=71)
    t = to_dev(x, cfg.dtype)
    O, Wf = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                              t["W_target"], cfg.eta, C, schedule=schedule)
    torch.cuda.synchronize()
    O, Wf = O.float().cpu().numpy(), Wf.cpu().numpy()
    O_ref, W_ref = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                                   x["W_target"], cfg.eta, C)
    W0 = np.broadcast_to(np.asarray(x["W_down0"], np.float64), W_ref.shape)
    e_o, e_dw = rel(O, O_ref), rel(Wf - W0, W_ref - W0)
    # The error of every sequence's state, so that a tile written to the
    # wrong sequence or region cannot hide behind the others.
    e_b = [rel(Wf[b] - W0[b], W_ref[b] - W0[b]) for b in range(B)]
    print(f"{case} {schedule}: O {e_o:.2e}  dW {e_dw:.2e}  per sequence "
          + " ".join(f"{e:.1e}" for e in e_b), flush=True)
    assert e_o <= O_TOL, f"O error {e_o:.3e}"
    assert max(e_b) <= DW_TOL, f"dW error {max(e_b):.3e}"


def test_packed_update_tilings_match_oracle(ttt):
    """The packed-document update at the Qwen3-4B widths (380 regions: 256
    wide tiles, then 124 regions as narrow pairs), with a document reset
    inside a chunk-aligned block sequence."""
    cfg = BASE.with_(name="packed_tilings", batch=1, seq_len=512, chunk=128, d_model=2560,
                     d_ff=9728)
    x = synth.make_inputs(cfg, seed=73)
    t = to_dev(x, cfg.dtype)
    starts = [0, 128, 320]
    O, Wf = ttt.layer_forward_packed(t["H"][0], t["X0"][0], t["Wg"], t["Wu"], t["W_down0"],
                                     t["taps"], t["W_target"], cfg.eta, cfg.chunk, starts)
    torch.cuda.synchronize()
    O, Wf = O.float().cpu().numpy(), Wf.cpu().numpy()
    O_ref, W_ref = ora.ttt_prefill_packed(x["H"][0], x["X0"][0], x["Wg"], x["Wu"],
                                          x["W_down0"], x["taps"], x["W_target"], cfg.eta,
                                          cfg.chunk, starts)
    W0 = np.asarray(x["W_down0"], np.float64)
    e_o, e_dw = rel(O, O_ref), rel(Wf - W0, W_ref - W0)
    print(f"packed tilings: O {e_o:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL and e_dw <= DW_TOL
