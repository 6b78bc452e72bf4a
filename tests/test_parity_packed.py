"""GPU parity for packed documents (ttt_layer_forward_packed) against the
CPU oracle's ttt_prefill_packed: the state returns to W_down0 at every
document start, chunks restart there, and the conv stops at the document
end (iplexlaw explainer §6). Tolerances as in test_parity.py."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as ora
import synth
from test_parity import DW_TOL, O_TOL, W_TOL, check_whole_sequence, rel, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import test_layer_gate_amd as m
    m.lib()
    return m


def run_packed_gpu(ttt, t, eta, chunk, starts, **kw):
    O, Wf = ttt.layer_forward_packed(t["H"][0], t["X0"][0], t["Wg"], t["Wu"], t["W_down0"],
                                     t["taps"], t["W_target"], eta, chunk, starts, **kw)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), Wf.cpu().numpy()


def check_packed(x, O, Wf, eta, chunk, starts, pad="sequence", raw_w=True):
    O_ref, W_ref = ora.ttt_prefill_packed(x["H"][0], x["X0"][0], x["Wg"], x["Wu"],
                                          x["W_down0"], x["taps"], x["W_target"], eta, chunk,
                                          starts, pad=pad)
    W0 = np.asarray(x["W_down0"], np.float64)
    e_o, e_w, e_dw = rel(O, O_ref), rel(Wf, W_ref), rel(Wf - W0, W_ref - W0)
    print(f"docs {starts[:6]}{'...' if len(starts) > 6 else ''}: "
          f"O {e_o:.2e}  W {e_w:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL, f"O error {e_o:.3e}"
    assert e_dw <= DW_TOL, f"dW error {e_dw:.3e}"
    if raw_w:
        assert e_w <= W_TOL, f"W error {e_w:.3e}"


DOCS = {
    "mixed": [0, 512, 576, 1344],          # 2 chunks, 64 tokens, 3 chunks, 2.75 chunks
    "one_chunk_each": list(range(0, 2048, 256)),
    "tiny_docs": list(range(0, 2048, 64)),  # 32 documents shorter than a chunk
}


@pytest.mark.parametrize("schedule", ["prefix", "running"])
@pytest.mark.parametrize("pad", ["sequence", "chunk"])
@pytest.mark.parametrize("docs", sorted(DOCS))
def test_packed_matches_oracle(ttt, docs, pad, schedule):
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=1)
    O, Wf = run_packed_gpu(ttt, to_dev(x, cfg.dtype), cfg.eta, cfg.chunk, DOCS[docs],
                           schedule=schedule, pad=pad)
    check_packed(x, O, Wf, cfg.eta, cfg.chunk, DOCS[docs], pad=pad)


def test_packed_ragged_fp32(ttt):
    """fp32 inputs, T = 1000 (the last document ragged), chunk 128."""
    cfg = synth.CONFIGS["tiny_amp"]
    x = synth.make_inputs(cfg, batch=1, seq_len=1000, seed=11)
    starts = [0, 320, 640]
    for schedule in ("prefix", "running"):
        O, Wf = run_packed_gpu(ttt, to_dev(x, cfg.dtype), cfg.eta, 128, starts,
                               schedule=schedule)
        check_packed(x, O, Wf, cfg.eta, 128, starts)


def test_single_document_is_the_plain_layer(ttt):
    """One document covering the sequence runs the same kernels as
    ttt_layer_forward with the same tiles: the results are bit-identical."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=1)
    t = to_dev(x, cfg.dtype)
    O_p, W_p = run_packed_gpu(ttt, t, cfg.eta, cfg.chunk, [0])
    O, W = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                             t["W_target"], cfg.eta, cfg.chunk)
    torch.cuda.synchronize()
    assert np.array_equal(O_p, O[0].float().cpu().numpy())
    assert np.array_equal(W_p, W[0].cpu().numpy())


def test_documents_do_not_leak(ttt):
    """Changing the tokens of one document leaves every output of the other
    documents bit-identical (reset forwards, conv boundary backwards)."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=1)
    starts = [0, 768, 1280]
    O, _ = run_packed_gpu(ttt, to_dev(x, cfg.dtype), cfg.eta, cfg.chunk, starts)
    y = dict(x, H=x["H"].copy(), X0=x["X0"].copy())
    y["H"][0, 768:1280] = synth.round_to_bf16(-y["H"][0, 768:1280])
    y["X0"][0, 768:1280] = synth.round_to_bf16(2 * y["X0"][0, 768:1280])
    O2, _ = run_packed_gpu(ttt, to_dev(y, cfg.dtype), cfg.eta, cfg.chunk, starts)
    assert np.array_equal(O[:768], O2[:768])
    assert np.array_equal(O[1280:], O2[1280:])
    assert not np.array_equal(O[768:1280], O2[768:1280])


@pytest.mark.timeout(900)
def test_packed_full_size_five_documents(ttt):
    """Qwen3-4B shape at 64k tokens, five documents of uneven lengths (some
    not multiples of the chunk): every output of every document against the
    oracle run on that document alone (packed documents equal separate runs,
    pinned in oracle_pins.py), and every entry of the final state, the last
    document's. tests/test_packed_tables.py checks this layout's step flags
    and snapshot slots on the CPU."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    x = synth.make_inputs(cfg)
    C, eta = cfg.chunk, cfg.eta
    starts = [0, 20480, 21568, 45056, 63488]
    print(f"[packed 64k] documents {starts}", flush=True)
    t = to_dev(x, cfg.dtype)
    O, Wf = run_packed_gpu(ttt, t, eta, C, starts)
    del t
    torch.cuda.empty_cache()
    bounds = starts + [cfg.seq_len]
    for a, e in zip(bounds[:-1], bounds[1:]):
        doc = {k: (v[:, a:e] if k in ("H", "X0") else v) for k, v in x.items()}
        print(f"[packed 64k] oracle on document [{a}, {e})", flush=True)
        check_whole_sequence(doc, O[None, a:e], Wf[None], eta, C, f"document [{a}, {e})",
                             check_state=e == cfg.seq_len)


@pytest.mark.timeout(900)
def test_packed_full_size_equal_documents_sampled(ttt):
    """Qwen3-4B shape at 64k tokens as 32 documents of 2048 tokens (two
    chunks each), the layout bench.py --variant packed times. Checked on
    whole documents the oracle runs alone (the first, one in the middle and
    the last: each second chunk sees its own first chunk's update and nothing
    of the document before) and on sampled entries of the final state (the
    last document's update on top of W_down0)."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    x = synth.make_inputs(cfg)
    C, eta, L = cfg.chunk, cfg.eta, 2048
    starts = list(range(0, cfg.seq_len, L))
    t = to_dev(x, cfg.dtype)
    O, Wf = run_packed_gpu(ttt, t, eta, C, starts)
    del t
    torch.cuda.empty_cache()
    one = {k: x[k] for k in ("Wg", "Wu", "W_down0", "taps", "W_target")}
    for a in (0, 13 * L, starts[-1]):
        O_ref, _ = ora.ttt_prefill(x["H"][:, a:a + L], x["X0"][:, a:a + L], one["Wg"],
                                   one["Wu"], one["W_down0"], one["taps"], one["W_target"],
                                   eta, C)
        eo = rel(O[a:a + L], O_ref[0])
        e2 = rel(O[a + C:a + L], O_ref[0, C:])
        print(f"document [{a}, {a + L}): O {eo:.2e}, second chunk {e2:.2e}", flush=True)
        assert eo <= O_TOL and e2 <= O_TOL
    rng = np.random.default_rng(98)
    cs = np.unique(np.concatenate([[0, cfg.d_model - 1], rng.integers(0, cfg.d_model, 14)]))
    js = np.unique(np.concatenate([[0, cfg.d_ff - 1], rng.integers(0, cfg.d_ff, 14)]))
    a = starts[-1]
    W_ref = ora.final_state_entries(x["H"][0, a:], x["X0"][0, a:], one["Wg"], one["Wu"],
                                    one["W_down0"], one["taps"], one["W_target"], eta, cs, js)
    W0s = x["W_down0"][np.ix_(cs, js)].astype(np.float64)
    W_s = Wf[np.ix_(cs, js)]
    ew, edw = rel(W_s, W_ref), rel(W_s - W0s, W_ref - W0s)
    print(f"final state after the last document: W {ew:.2e} dW {edw:.2e}", flush=True)
    assert ew <= W_TOL and edw <= DW_TOL


def test_packed_at_the_step_limit(ttt):
    """131072 tokens, the longest packed sequence (2048 update steps of 64
    tokens, the last one held by the last bit of the update's per-lane step
    registers), with documents that put a chunk start inside a document at
    step 2044 and a document start on step 2047; mid_amp widths, chunk 256.
    Every output against the oracle, and the final state, which is the last
    one-step document's update on W_down0."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, batch=1, seq_len=131072, seed=59)
    starts = [0, 640, 65536, 130560, 131008]
    O, Wf = run_packed_gpu(ttt, to_dev(x, cfg.dtype), cfg.eta, cfg.chunk, starts)
    check_packed(x, O, Wf, cfg.eta, cfg.chunk, starts)
