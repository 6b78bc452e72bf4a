"""GPU parity for the decode step (ttt_decode_begin / ttt_decode_step): one
token per sequence at a time, with chunk-local padding, against the CPU
oracle's ttt_decode (itself pinned to the chunk-padded prefill). Tolerances
as in test_parity.py."""
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


def new_state(ttt, t, B, chunk, W_state):
    desc = ttt.make_desc(B, 1, t["Wg"].shape[1], t["Wg"].shape[0], t["taps"].shape[0],
                         1 if t["H"].dtype == torch.float32 else 0,
                         1 if t["Wg"].dtype == torch.float32 else 0, 0,
                         ttt._binding.FLAG_PAD_CHUNK)
    ds = torch.empty(ttt.decode_state_size(desc, chunk), dtype=torch.uint8, device="cuda")
    ttt.decode_begin(W_state, chunk, ds, act_dtype=t["H"].dtype, weight_dtype=t["Wg"].dtype,
                     conv_k=t["taps"].shape[0])
    return ds


def decode_gpu(ttt, t, eta, chunk, a, e, W_state):
    """Decodes tokens [a, e) of every sequence (a a multiple of chunk) from
    W_state (updated in place); returns O [B, e - a, d] on the host."""
    B = t["H"].shape[0]
    ds = new_state(ttt, t, B, chunk, W_state)
    outs = []
    for pos in range(a, e):
        h = t["H"][:, pos].contiguous()
        x0 = t["X0"][:, pos].contiguous()
        outs.append(ttt.decode_step(h, x0, t["Wg"], t["Wu"], t["taps"], t["W_target"], eta,
                                    chunk, pos, W_state, ds))
    torch.cuda.synchronize()
    return torch.stack(outs, dim=1).float().cpu().numpy()


def state0(t, B):
    W = t["W_down0"].float()
    return (W.expand(B, *W.shape) if W.dim() == 2 else W).contiguous().clone()


def check(x, O, W, eta, chunk, what, raw_w=True, a=0, W_in=None):
    W0 = x["W_down0"] if W_in is None else W_in
    O_ref, W_ref, pending = ora.ttt_decode(x["H"][:, a:], x["X0"][:, a:], x["Wg"], x["Wu"], W0,
                                           x["taps"], x["W_target"], eta, chunk, start=a)
    W0b = np.broadcast_to(np.asarray(W0, np.float64), W_ref.shape)
    e_o, e_w, e_dw = rel(O, O_ref), rel(W, W_ref), rel(W - W0b, W_ref - W0b)
    print(f"{what}: O {e_o:.2e}  W {e_w:.2e}  dW {e_dw:.2e}  pending {pending}", flush=True)
    assert e_o <= O_TOL, f"O error {e_o:.3e}"
    assert e_dw <= DW_TOL, f"dW error {e_dw:.3e}"
    if raw_w:
        assert e_w <= W_TOL, f"W error {e_w:.3e}"
    return pending


@pytest.mark.parametrize("name,B,T", [("mid_amp", 1, 1024), ("mid_amp", 2, 1000),
                                      ("mid_amp", 10, 300),  # past one pass of 8 sequences
                                      ("tiny", 2, 256), ("tiny_amp", 1, 200)])
def test_decode_matches_oracle(ttt, name, B, T):
    """Whole sequences decoded token by token: every output, and the state
    after the last whole chunk (a ragged end leaves its chunk pending)."""
    cfg = synth.CONFIGS[name]
    x = synth.make_inputs(cfg, batch=B, seq_len=T, seed=31 + T)
    t = to_dev(x, cfg.dtype)
    W = state0(t, B)
    O = decode_gpu(ttt, t, cfg.eta, cfg.chunk, 0, T, W)
    pending = check(x, O, W.cpu().numpy(), cfg.eta, cfg.chunk, f"{name} B={B} T={T}")
    assert pending == T % cfg.chunk


def test_decode_continues_a_prefill(ttt):
    """Prefill of two chunks (chunk-padded, through ttt_layer_forward_continue),
    then decode of the rest from the state it returned: the one chunk-padded
    prefill's outputs and final state."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, seq_len=1024, seed=41)
    t = to_dev(x, cfg.dtype)
    C, eta, a = cfg.chunk, cfg.eta, 512
    W = state0(t, 1)
    O1 = ttt.layer_forward_continue(t["H"][:, :a].contiguous(), t["X0"][:, :a].contiguous(),
                                    None, t["Wg"], t["Wu"], W, t["taps"], t["W_target"], eta,
                                    C, pad="chunk")
    O2 = decode_gpu(ttt, t, eta, C, a, 1024, W)
    O = np.concatenate([O1.float().cpu().numpy(), O2], axis=1)
    O_ref, W_ref = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                                   x["W_target"], eta, C, pad="chunk")
    W0 = np.asarray(x["W_down0"], np.float64)
    e_o, e_dw = rel(O, O_ref), rel(W.cpu().numpy() - W0, W_ref - W0)
    print(f"prefill + decode: O {e_o:.2e}  dW {e_dw:.2e}", flush=True)
    assert e_o <= O_TOL and e_dw <= DW_TOL


def test_decode_agrees_with_the_gpu_prefill(ttt):
    """Decode and the chunk-padded prefill on the GPU round the same values
    (Z, V, the bf16 state copies) and differ only in summation order."""
    cfg = synth.CONFIGS["mid_amp"]
    x = synth.make_inputs(cfg, seq_len=768, seed=43)
    t = to_dev(x, cfg.dtype)
    W = state0(t, 1)
    O = decode_gpu(ttt, t, cfg.eta, cfg.chunk, 0, 768, W)
    Op, Wp = ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                               t["W_target"], cfg.eta, cfg.chunk, pad="chunk")
    torch.cuda.synchronize()
    Wp = Wp.cpu().numpy()
    e_o, e_w = rel(O, Op.float().cpu().numpy()), rel(W.cpu().numpy(), Wp)
    print(f"decode vs prefill on the GPU: O {e_o:.2e}  W {e_w:.2e}", flush=True)
    assert e_o <= 1e-2 and e_w <= 1e-4


@pytest.mark.timeout(900)
def test_decode_full_size_sampled(ttt):
    """Qwen3-4B shape, 1030 tokens decoded: the first chunk against the
    incoming state, the 6 tokens of the second against the state after the
    first chunk's update, and sampled entries of that state."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    T, C, eta = 1030, cfg.chunk, cfg.eta
    x = synth.make_inputs(cfg, seq_len=T, seed=47)
    t = to_dev(x, cfg.dtype)
    W = state0(t, 1)
    O = decode_gpu(ttt, t, eta, C, 0, T, W)[0]
    Wg = W[0].cpu().numpy()
    del t, W
    torch.cuda.empty_cache()
    O_ref, _ = ora.ttt_prefill(x["H"], x["X0"], x["Wg"], x["Wu"], x["W_down0"], x["taps"],
                               x["W_target"], eta, C, pad="chunk")
    e_o1, e_o2 = rel(O[:C], O_ref[0, :C]), rel(O[C:], O_ref[0, C:])
    rng = np.random.default_rng(97)
    cs = np.unique(np.concatenate([[0, cfg.d_model - 1], rng.integers(0, cfg.d_model, 14)]))
    js = np.unique(np.concatenate([[0, cfg.d_ff - 1], rng.integers(0, cfg.d_ff, 14)]))
    W_ref = ora.final_state_entries(x["H"][0, :C], x["X0"][0, :C], x["Wg"], x["Wu"],
                                    x["W_down0"], x["taps"], x["W_target"], eta, cs, js,
                                    pad="chunk", chunk=C)
    W0s = x["W_down0"][np.ix_(cs, js)].astype(np.float64)
    W_s = Wg[np.ix_(cs, js)]
    ew, edw = rel(W_s, W_ref), rel(W_s - W0s, W_ref - W0s)
    print(f"decode 64k shape: O first chunk {e_o1:.2e}, second {e_o2:.2e}; "
          f"state W {ew:.2e} dW {edw:.2e}", flush=True)
    assert e_o1 <= O_TOL and e_o2 <= O_TOL and ew <= W_TOL and edw <= DW_TOL
