"""Pins for the CPU oracle: checks against things other than the oracle.

Every pin computes its expected side without the oracle's code: with torch's
CPU library routines (silu, conv1d, matmul), with brute-force scalar loops,
with the closed forms the pages give (next-token target), or with an
invariant of the method (linearity in eta, chunk causality, batch
independence, split/resume, the prefix-scan and state-free forms). Each pin
raises AssertionError when the oracle disagrees. They are plain functions so
that tests/test_oracle_mutations.py can rerun them against an oracle with a
planted mistake and check that some pin fails.

Page citations use the keys of the oracle's header: [notes] reading notes,
[forum] zhichai summary, [iplex] iplexlaw explainer.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.ttt_oracle as ora

RTOL = 1e-10


def _close(a, b, tol=RTOL, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(np.abs(b).max(), 1e-300)
    err = np.abs(a - b).max() / scale
    assert err <= tol, f"{what}: max|err|/max|ref| = {err:.3e} > {tol:.1e}"


def small_case(seed=0, B=2, T=37, d=6, f=10, K=3, C=8, eta=0.05,
               x0_std=1.0, wt_std=0.4):
    """Small float64 inputs whose fast-weight term is a large share of O."""
    rng = np.random.default_rng(seed)
    return dict(
        H=rng.standard_normal((B, T, d)),
        X0=rng.standard_normal((B, T, d)) * x0_std,
        Wg=rng.standard_normal((f, d)) / math.sqrt(d),
        Wu=rng.standard_normal((f, d)) / math.sqrt(d),
        W_down0=rng.standard_normal((d, f)) / math.sqrt(f),
        taps=rng.standard_normal((K, d)) / math.sqrt(K),
        W_target=rng.standard_normal((d, d)) * wt_std,
        eta=eta, chunk=C)


def run(x, **over):
    a = dict(x)
    a.update(over)
    kw = {"clip": a["clip"]} if a.get("clip") is not None else {}
    return ora.ttt_prefill(a["H"], a["X0"], a["Wg"], a["Wu"], a["W_down0"],
                           a["taps"], a["W_target"], a["eta"], a["chunk"],
                           pad=a.get("pad", "sequence"), **kw)


# ---- library-routine references (torch, CPU, float64) ----------------------

def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def torch_z(H_b, Wg, Wu):
    """Gated activation via torch.nn.functional.silu ([notes] gated MLP)."""
    Hb = _t(H_b)
    return (torch.nn.functional.silu(Hb @ _t(Wg).T) * (Hb @ _t(Wu).T)).numpy()


def torch_conv(X0_b, taps, pad="sequence", chunk=None):
    """Depthwise conv via torch conv1d (a cross-correlation, so output t
    reads inputs t .. t+K-1), right-padded with K-1 zeros."""
    K = taps.shape[0]
    w = _t(taps).T.unsqueeze(1)                           # [d, 1, K]

    def conv(rows):
        x = _t(rows).T.unsqueeze(0)                       # [1, d, n]
        x = torch.nn.functional.pad(x, (0, K - 1))
        return torch.nn.functional.conv1d(x, w, groups=x.shape[1])[0].T.numpy()

    if pad == "sequence":
        return conv(X0_b)
    T = X0_b.shape[0]
    return np.concatenate([conv(X0_b[a:min(a + chunk, T)])
                           for a in range(0, T, chunk)])


def torch_target(X0_b, taps, W_target, pad="sequence", chunk=None):
    return (_t(torch_conv(X0_b, taps, pad, chunk)) @ _t(W_target)).numpy()


def plain_mlp(H_b, Wg, Wu, W0):
    return (_t(torch_z(H_b, Wg, Wu)) @ _t(W0).T).numpy()


# ---- pins -------------------------------------------------------------------

def pin_reduces_to_plain_mlp():
    """eta = 0, zero taps, W_target = 0, or one chunk covering the sequence:
    the output is the plain gated MLP ([notes] gated-MLP equation); the final
    state is W_down0, or W_down0 + eta V^T Z for the single chunk."""
    x = small_case(seed=1)
    ref = np.stack([plain_mlp(x["H"][b], x["Wg"], x["Wu"], x["W_down0"])
                    for b in range(2)])
    for over in ({"eta": 0.0}, {"taps": np.zeros_like(x["taps"])},
                 {"W_target": np.zeros_like(x["W_target"])}):
        O, Wf = run(x, **over)
        _close(O, ref, what=f"plain MLP {list(over)}")
        for b in range(2):
            _close(Wf[b], x["W_down0"], what=f"W_final {list(over)}")
    O, Wf = run(x, chunk=64)
    _close(O, ref, what="single chunk")
    for b in range(2):
        Z = torch_z(x["H"][b], x["Wg"], x["Wu"])
        V = torch_target(x["X0"][b], x["taps"], x["W_target"])
        _close(Wf[b], x["W_down0"] + x["eta"] * V.T @ Z, what="single-chunk W")


def pin_prefix_scan_form():
    """The sequential recurrence equals the three-step form of [iplex] §6:
    all chunk deltas, an exclusive prefix sum, then every chunk's output
    with W_down0 + eta * prefix. Z and V come from torch here."""
    for pad in ("sequence", "chunk"):
        x = small_case(seed=2, T=41, C=8)
        O, Wf = run(x, pad=pad)
        for b in range(2):
            Z = torch_z(x["H"][b], x["Wg"], x["Wu"])
            V = torch_target(x["X0"][b], x["taps"], x["W_target"], pad, 8)
            starts = list(range(0, 41, 8))
            deltas = np.stack([V[s:s + 8].T @ Z[s:s + 8] for s in starts])
            prefix = np.cumsum(deltas, axis=0) - deltas          # exclusive
            for i, s in enumerate(starts):
                W_i = x["W_down0"] + x["eta"] * prefix[i]
                _close(O[b, s:s + 8], Z[s:s + 8] @ W_i.T,
                       what=f"prefix form O chunk {i} ({pad})")
            _close(Wf[b], x["W_down0"] + x["eta"] * deltas.sum(0),
                   what=f"prefix form W_final ({pad})")


def pin_state_free_form():
    """Unrolling the update gives, for token t in chunk i,
    O_t = W_down0 Z_t + eta * sum_{s before chunk i} (Z_s . Z_t) V_s,
    computed here token by token with no state."""
    x = small_case(seed=3, T=29, C=6)
    O, _ = run(x)
    for b in range(2):
        Z = torch_z(x["H"][b], x["Wg"], x["Wu"])
        V = torch_target(x["X0"][b], x["taps"], x["W_target"])
        for t in range(29):
            first = (t // 6) * 6
            o = x["W_down0"] @ Z[t]
            for s in range(first):
                o = o + x["eta"] * float(Z[s] @ Z[t]) * V[s]
            _close(O[b, t], o, tol=1e-9, what=f"state-free O[{b},{t}]")


def pin_next_token_target():
    """taps = [0, 1, 0, ...] with W_target = I makes the target the next
    token's embedding ([forum] design 3): V_t = X0[t + 1], zero past the end;
    with chunk padding also zero at each chunk's last token."""
    rng = np.random.default_rng(4)
    T, d, K, C = 19, 5, 4, 6
    X0 = rng.standard_normal((T, d))
    taps = np.zeros((K, d))
    taps[1] = 1.0
    V = ora.lm_target(X0, taps, np.eye(d))
    for t in range(T):
        want = X0[t + 1] if t + 1 < T else np.zeros(d)
        assert np.array_equal(V[t], want), f"NTP row {t}"
    V = ora.lm_target(X0, taps, np.eye(d), pad="chunk", chunk=C)
    for t in range(T):
        nxt = t + 1
        want = X0[nxt] if (nxt < T and nxt // C == t // C) else np.zeros(d)
        assert np.array_equal(V[t], want), f"NTP chunk-padded row {t}"


def pin_conv_library():
    """The conv and projection match torch conv1d (both paddings) and a
    non-square orientation check of W_target."""
    rng = np.random.default_rng(5)
    X0 = rng.standard_normal((23, 7))
    taps = rng.standard_normal((4, 7))
    Wt = rng.standard_normal((7, 7))
    _close(ora.conv_target_input(X0, taps), torch_conv(X0, taps), what="conv")
    _close(ora.conv_target_input(X0, taps, "chunk", 5),
           torch_conv(X0, taps, "chunk", 5), what="chunk conv")
    _close(ora.lm_target(X0, taps, Wt), torch_target(X0, taps, Wt),
           what="target")
    _close(ora.lm_target(X0, taps, Wt, "chunk", 5),
           torch_target(X0, taps, Wt, "chunk", 5), what="chunk target")


def pin_linear_in_eta():
    """O and W_final are affine in eta: the update adds eta times a quantity
    that does not depend on eta, so hidden normalisation or clipping shows."""
    x = small_case(seed=6)
    O0, W0 = run(x, eta=0.0)
    O1, W1 = run(x, eta=0.03)
    O3, W3 = run(x, eta=0.09)
    _close(O3 - O0, 3.0 * (O1 - O0), tol=1e-9, what="O linear in eta")
    _close(W3 - W0, 3.0 * (W1 - W0), tol=1e-9, what="W linear in eta")
    assert np.abs(O1 - O0).max() > 1e-3 * np.abs(O0).max(), "fast term vanished"


def pin_chunk_causality():
    """[iplex] §3: a chunk's output uses only earlier chunks. Changing H in
    chunk j leaves every earlier output bitwise unchanged, and changes chunk
    j + 1. Changing X0 in chunk j leaves outputs before chunk j unchanged;
    with chunk padding, also chunk j's own output."""
    x = small_case(seed=7, T=40, C=8)
    O, _ = run(x)
    j = 2
    for key in ("H", "X0"):
        y = dict(x)
        y[key] = x[key].copy()
        y[key][:, j * 8:(j + 1) * 8] += 1.0
        O2, _ = run(y)
        assert np.array_equal(O2[:, :j * 8], O[:, :j * 8]), f"{key} leaked back"
        assert not np.allclose(O2[:, (j + 1) * 8:(j + 2) * 8],
                               O[:, (j + 1) * 8:(j + 2) * 8]), f"{key} unused"
    Oc, _ = run(x, pad="chunk")
    y = dict(x)
    y["X0"] = x["X0"].copy()
    y["X0"][:, j * 8:(j + 1) * 8] += 1.0
    O2, _ = run(y, pad="chunk")
    assert np.array_equal(O2[:, :(j + 1) * 8], Oc[:, :(j + 1) * 8]), \
        "chunk padding leaked"


def pin_batch_independence():
    """[iplex] §6: state is per document. A batch of two equals two calls of
    one, with a shared or a per-sequence W_down0."""
    x = small_case(seed=8)
    O, Wf = run(x)
    for b in range(2):
        Ob, Wb = run(x, H=x["H"][b:b + 1], X0=x["X0"][b:b + 1])
        _close(O[b:b + 1], Ob, tol=1e-14, what="batch O")
        _close(Wf[b:b + 1], Wb, tol=1e-14, what="batch W")
    W0b = np.stack([x["W_down0"], 2.0 * x["W_down0"]])
    O, Wf = run(x, W_down0=W0b)
    Ob, Wb = run(x, H=x["H"][1:], X0=x["X0"][1:], W_down0=2.0 * x["W_down0"])
    _close(O[1:], Ob, tol=1e-14, what="per-sequence W_down0 O")
    _close(Wf[1:], Wb, tol=1e-14, what="per-sequence W_down0 W")


def pin_split_resume():
    """Running chunks [0, j) with K - 1 look-ahead rows of X0, then the rest
    from the returned state, reproduces the single run."""
    x = small_case(seed=9, T=45, C=8, K=3)
    O, Wf = run(x)
    cut = 3 * 8
    O1, W1 = run(x, H=x["H"][:, :cut], X0=x["X0"][:, :cut + 2])
    O2, W2 = run(x, H=x["H"][:, cut:], X0=x["X0"][:, cut:], W_down0=W1)
    _close(np.concatenate([O1, O2], axis=1), O, tol=1e-12, what="split O")
    _close(W2, Wf, tol=1e-12, what="split W")


def pin_brute_force_scalars():
    """Every quantity by scalar loops in Python floats, math.exp for the
    sigmoid, on a ragged sequence (T = 7, C = 3: chunks of 3, 3, 1)."""
    x = small_case(seed=10, B=1, T=7, d=3, f=4, K=2, C=3, eta=0.2)
    O, Wf = run(x)
    H, X0 = x["H"][0].tolist(), x["X0"][0].tolist()
    Wg, Wu, W = x["Wg"].tolist(), x["Wu"].tolist(), x["W_down0"].tolist()
    taps, Wt = x["taps"].tolist(), x["W_target"].tolist()
    T, d, f, K, C, eta = 7, 3, 4, 2, 3, 0.2
    Z = [[0.0] * f for _ in range(T)]
    for t in range(T):
        for j in range(f):
            g = sum(H[t][c] * Wg[j][c] for c in range(d))
            u = sum(H[t][c] * Wu[j][c] for c in range(d))
            Z[t][j] = g / (1.0 + math.exp(-g)) * u
    V = [[0.0] * d for _ in range(T)]
    for t in range(T):
        y = [sum(taps[k][c] * X0[t + k][c] for k in range(K) if t + k < T)
             for c in range(d)]
        for o in range(d):
            V[t][o] = sum(y[c] * Wt[c][o] for c in range(d))
    W = [row[:] for row in W]
    want = [[0.0] * d for _ in range(T)]
    for start in range(0, T, C):
        end = min(start + C, T)
        for t in range(start, end):
            for o in range(d):
                want[t][o] = sum(Z[t][j] * W[o][j] for j in range(f))
        for o in range(d):
            for j in range(f):
                W[o][j] += eta * sum(V[t][o] * Z[t][j] for t in range(start, end))
    _close(O[0], want, tol=1e-12, what="scalar O")
    _close(Wf[0], W, tol=1e-12, what="scalar W")


def pin_sampled_forms():
    """The sampled helpers used at full size agree with the full recurrence
    and with torch."""
    x = small_case(seed=11, T=33, C=8)
    for pad in ("sequence", "chunk"):
        _, Wf = run(x, pad=pad)
        cs, js = [0, 3, 5], [1, 2, 9]
        for b in range(2):
            got = ora.final_state_entries(x["H"][b], x["X0"][b], x["Wg"],
                                          x["Wu"], x["W_down0"], x["taps"],
                                          x["W_target"], x["eta"], cs, js,
                                          pad=pad, chunk=8)
            _close(got, Wf[b][np.ix_(cs, js)], tol=1e-12,
                   what=f"final entries ({pad})")
            rows = [0, 7, 8, 31, 32]
            _close(ora.target_rows(x["X0"][b], x["taps"], x["W_target"], rows,
                                   pad=pad, chunk=8),
                   torch_target(x["X0"][b], x["taps"], x["W_target"], pad, 8)[rows],
                   what=f"target rows ({pad})")
    # a segment whose X0 carries two look-ahead rows past its 24 tokens
    _, W1 = run(x, H=x["H"][:, :24], X0=x["X0"][:, :26])
    for b in range(2):
        got = ora.final_state_entries(x["H"][b, :24], x["X0"][b, :26], x["Wg"], x["Wu"],
                                      x["W_down0"], x["taps"], x["W_target"], x["eta"],
                                      [0, 3, 5], [1, 2, 9])
        _close(got, W1[b][np.ix_([0, 3, 5], [1, 2, 9])], tol=1e-12,
               what="final entries (look-ahead)")
    _close(ora.activation_rows(x["H"][0], x["Wg"], x["Wu"], [2, 30]),
           torch_z(x["H"][0], x["Wg"], x["Wu"])[[2, 30]], what="Z rows")


def pin_golden_ntp_fixture():
    """The hand-written next-token example in tests/golden/ntp_shift.txt."""
    import pathlib
    p = pathlib.Path(__file__).parent / "golden" / "ntp_shift.txt"
    blocks = {}
    cur = None
    for line in p.read_text().splitlines():
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            cur = line[:-1]
            blocks[cur] = []
        else:
            blocks[cur].append([float(v) for v in line.split()])
    X0 = np.array(blocks["X0"])
    taps = np.array(blocks["taps"])
    V = ora.lm_target(X0, taps, np.eye(X0.shape[1]))
    assert np.array_equal(V, np.array(blocks["V_expected"])), "golden NTP"


# ---- update-norm clipping ([iplex] §6) ---------------------------------------

def pin_clip_loose_is_plain():
    """A limit no chunk's update reaches changes nothing."""
    x = small_case(seed=31)
    O, W = run(x)
    O2, W2 = run(x, clip=1e12)
    assert np.array_equal(O, O2) and np.array_equal(W, W2), "loose clip changed the result"


def pin_clip_each_delta():
    """Each chunk's applied update, read off the states after successive
    chunks (the prefill of the first j chunks, with the conv's K - 1
    look-ahead rows), is the torch-computed eta V_j^T Z_j scaled to norm
    min(||eta V_j^T Z_j||_F, clip): same direction, clipped length."""
    x = small_case(seed=32, B=1, T=40, C=8, eta=0.3)
    K, C, T = x["taps"].shape[0], x["chunk"], 40
    Z = torch_z(x["H"][0], x["Wg"], x["Wu"])
    V = torch_target(x["X0"][0], x["taps"], x["W_target"])
    raw = [x["eta"] * (_t(V[a:a + C]).T @ _t(Z[a:a + C])).numpy() for a in range(0, T, C)]
    norms = [float(np.linalg.norm(r)) for r in raw]
    clip = float(np.median(norms))            # clips about half of the chunks
    prev = np.asarray(x["W_down0"], np.float64)
    for j, a in enumerate(range(0, T, C)):
        n = min(a + C, T)
        sub = dict(x, H=x["H"][:, :n], X0=x["X0"][:, :n + K - 1])
        _, Wj = run(sub, clip=clip)
        delta = Wj[0] - prev
        want = raw[j] * min(1.0, clip / norms[j])
        _close(delta, want, tol=1e-9, what=f"clipped delta of chunk {j}")
        prev = Wj[0]


# ---- packed documents ([iplex] §6, reset at document boundaries) ----------

PACKED_DOCS = ([0, 13, 30, 31], [0, 8, 24], [0, 20])  # lengths below, at and above C = 8


def run_packed(x, starts, pad="sequence", b=0, clip=None):
    kw = {"clip": clip} if clip is not None else {}
    return ora.ttt_prefill_packed(x["H"][b], x["X0"][b], x["Wg"], x["Wu"], x["W_down0"],
                                  x["taps"], x["W_target"], x["eta"], x["chunk"], starts,
                                  pad=pad, **kw)


def pin_packed_single_document():
    """One document covering the sequence is the plain prefill of that
    sequence (the packed form is written token by token, the plain one chunk
    by chunk)."""
    x = small_case(seed=21, B=1, T=29)
    for pad in ("sequence", "chunk"):
        O, W = run_packed(x, [0], pad)
        O_ref, W_ref = run(x, pad=pad)
        _close(O, O_ref[0], what=f"packed single O ({pad})")
        _close(W, W_ref[0], what=f"packed single W ({pad})")


def pin_packed_equals_documents():
    """[iplex] §6: a packed sequence equals its documents run one by one from
    W_down0, each on its own tokens only (no look-ahead into the next
    document); the returned state is the last document's."""
    x = small_case(seed=22, B=1, T=40)
    for starts in PACKED_DOCS:
        for pad in ("sequence", "chunk"):
            O, W = run_packed(x, starts, pad)
            bounds = list(starts) + [40]
            for a, e in zip(bounds, bounds[1:]):
                sub = dict(x, H=x["H"][:, a:e], X0=x["X0"][:, a:e])
                O_ref, W_ref = run(sub, pad=pad)
                _close(O[a:e], O_ref[0], what=f"document [{a},{e}) O ({pad})")
            _close(W, W_ref[0], what=f"final state after {starts} ({pad})")


def pin_packed_clip_equals_documents():
    """Packed documents with update-norm clipping equal the documents run one
    by one through the clipped prefill (itself pinned chunk by chunk by
    pin_clip_each_delta), at a limit between the chunks' update norms (the
    median of the torch-computed norms), so that some chunks are clipped and
    some are not."""
    x = small_case(seed=24, B=1, T=40, eta=0.3)
    C = x["chunk"]
    starts = [0, 13, 30]
    bounds = starts + [40]
    norms = []
    for a, e in zip(bounds, bounds[1:]):
        Z = torch_z(x["H"][0, a:e], x["Wg"], x["Wu"])
        V = torch_target(x["X0"][0, a:e], x["taps"], x["W_target"])
        for c in range(0, e - a, C):
            norms.append(x["eta"] * float(torch.linalg.matrix_norm(
                _t(V[c:c + C]).T @ _t(Z[c:c + C]))))
    clip = float(np.median(norms))
    assert min(norms) < clip < max(norms)
    O, W = run_packed(x, starts, clip=clip)
    for a, e in zip(bounds, bounds[1:]):
        sub = dict(x, H=x["H"][:, a:e], X0=x["X0"][:, a:e])
        O_ref, W_ref = run(sub, clip=clip)
        _close(O[a:e], O_ref[0], what=f"clipped document [{a},{e}) O")
    _close(W, W_ref[0], what="clipped final state")
    _, W_free = run_packed(x, starts)
    assert not np.allclose(W, W_free), "the limit changed nothing"


def pin_packed_isolation():
    """No information crosses a document boundary in either direction:
    changing the tokens of one document changes no output of another (a
    missing reset leaks forwards; a conv read past the boundary leaks
    backwards)."""
    x = small_case(seed=23, B=1, T=40)
    starts = [0, 13, 30]
    O, _ = run_packed(x, starts)
    rng = np.random.default_rng(5)
    for a, e in ((0, 13), (13, 30), (30, 40)):
        y = dict(x, H=x["H"].copy(), X0=x["X0"].copy())
        y["H"][0, a:e] += rng.standard_normal((e - a, x["H"].shape[2]))
        y["X0"][0, a:e] += rng.standard_normal((e - a, x["X0"].shape[2]))
        O2, _ = run_packed(y, starts)
        keep = np.ones(40, bool)
        keep[a:e] = False
        assert np.array_equal(O[keep], O2[keep]), f"document [{a},{e}) leaked"
        assert not np.allclose(O[a:e], O2[a:e]), f"document [{a},{e}) ignored its input"


def decode(x, **over):
    a = dict(x)
    a.update(over)
    return ora.ttt_decode(a["H"], a["X0"], a["Wg"], a["Wu"], a["W_down0"], a["taps"],
                          a["W_target"], a["eta"], a["chunk"], start=a.get("start", 0))


def pin_decode_is_chunk_padded_prefill():
    """Token-by-token decode equals the chunk-padded prefill: every output,
    and the state after whole chunks (the sequence is 4 chunks long)."""
    x = small_case(seed=21, T=32, C=8)
    O, Wf = run(x, pad="chunk")
    Od, Wd, pending = decode(x)
    assert pending == 0
    _close(Od, O, tol=1e-12, what="decode O")
    _close(Wd, Wf, tol=1e-12, what="decode W")


def pin_decode_pending_chunk():
    """A ragged end: the outputs still match the prefill, but the state is
    the one after the last whole chunk (the prefill of those tokens alone)
    and the 5 tokens of the open chunk are pending."""
    x = small_case(seed=22, T=37, C=8)
    O, _ = run(x, pad="chunk")
    _, W32 = run(x, H=x["H"][:, :32], X0=x["X0"][:, :32], pad="chunk")
    Od, Wd, pending = decode(x)
    assert pending == 5
    _close(Od, O, tol=1e-12, what="ragged decode O")
    _close(Wd, W32, tol=1e-12, what="ragged decode W")


def pin_decode_resumes_prefill():
    """Prefill of the first two chunks, then decode from the state it
    returned, reproduces the single chunk-padded prefill."""
    x = small_case(seed=23, T=40, C=8)
    O, Wf = run(x, pad="chunk")
    O1, W1 = run(x, H=x["H"][:, :16], X0=x["X0"][:, :16], pad="chunk")
    O2, W2, pending = decode(x, H=x["H"][:, 16:], X0=x["X0"][:, 16:], W_down0=W1, start=16)
    assert pending == 0
    _close(np.concatenate([O1, O2], axis=1), O, tol=1e-12, what="prefill + decode O")
    _close(W2, Wf, tol=1e-12, what="prefill + decode W")


# ---- the backward pass -------------------------------------------------------

BWD_KEYS = ("H", "X0", "Wg", "Wu", "W_down0", "taps", "W_target")
GRAD_OF = {"H": "dH", "X0": "dX0", "Wg": "dWg", "Wu": "dWu", "W_down0": "dW_down0",
           "taps": "dtaps", "W_target": "dW_target"}


def backward_case(seed, per_seq=False, lookahead=0, **kw):
    """A small case for the backward: a ragged sequence, a batch of two, the
    upstream gradients dO and dW_final drawn too."""
    x = small_case(seed=seed, **kw)
    rng = np.random.default_rng(1000 + seed)
    B, T, d = x["H"].shape
    f = x["Wg"].shape[0]
    if lookahead:
        x["X0"] = np.concatenate([x["X0"], rng.standard_normal((B, lookahead, d))], axis=1)
    if per_seq:
        x["W_down0"] = rng.standard_normal((B, d, f)) / math.sqrt(f)
    x["dO"] = rng.standard_normal((B, T, d))
    x["dW_final"] = rng.standard_normal((B, d, f))
    return x


def backward(x, **over):
    a = dict(x)
    a.update(over)
    return ora.ttt_prefill_backward(a["H"], a["X0"], a["Wg"], a["Wu"], a["W_down0"],
                                    a["taps"], a["W_target"], a["eta"], a["chunk"], a["dO"],
                                    a.get("dW_final"), pad=a.get("pad", "sequence"))


def _loss(x, **over):
    """<dO, O> + <dW_final, W_final> through the forward oracle."""
    a = dict(x)
    a.update(over)
    O, Wf = run(a)
    return float((O * a["dO"]).sum() + (Wf * a["dW_final"]).sum())


def pin_backward_finite_differences():
    """Each gradient's directional derivative equals the central difference of
    the forward oracle's <dO, O> + <dW_final, W_final> along a random
    direction (float64, step 1e-6): both paddings, a shared and a
    per-sequence W_down0, look-ahead rows of X0, a ragged last chunk."""
    for seed, pad, per_seq, la in ((30, "sequence", False, 2), (31, "chunk", True, 0),
                                   (32, "sequence", True, 0)):
        x = backward_case(seed, per_seq=per_seq, lookahead=la, T=29, C=8)
        x["pad"] = pad
        g = backward(x)
        rng = np.random.default_rng(seed)
        for key in BWD_KEYS:
            v = rng.standard_normal(np.shape(x[key]))
            eps = 1e-6
            fd = (_loss(x, **{key: x[key] + eps * v}) - _loss(x, **{key: x[key] - eps * v})) \
                / (2 * eps)
            an = float((g[GRAD_OF[key]] * v).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
                f"{key} ({pad}): finite difference {fd:.12g} vs gradient {an:.12g}"


def _torch_prefill(t, eta, chunk, pad):
    """The prefill restated in torch (float64), for autograd: per sequence,
    the gated MLP with torch's silu, the conv as shifted sums over the reads
    before each token's bound, the chunk loop of apply then update."""
    H, X0, Wg, Wu, W0, taps, Wt = (t[k] for k in BWD_KEYS)
    B, T, d = H.shape
    T_in, K = X0.shape[1], taps.shape[0]
    Os, Ws = [], []
    for b in range(B):
        Z = torch.nn.functional.silu(H[b] @ Wg.T) * (H[b] @ Wu.T)
        rows = []
        for i in range(T):
            end = T_in if pad == "sequence" else min((i // chunk + 1) * chunk, T_in)
            y = torch.zeros(d, dtype=torch.float64)
            for k in range(K):
                if i + k < end:
                    y = y + taps[k] * X0[b, i + k]
            rows.append(y)
        V = torch.stack(rows) @ Wt
        W = W0[b] if W0.dim() == 3 else W0
        outs = []
        for a in range(0, T, chunk):
            outs.append(Z[a:a + chunk] @ W.T)
            W = W + eta * (V[a:a + chunk].T @ Z[a:a + chunk])
        Os.append(torch.cat(outs))
        Ws.append(W)
    return torch.stack(Os), torch.stack(Ws)


def pin_backward_autograd():
    """Every gradient equals torch autograd through a torch restatement of
    the forward (float64): both paddings, shared and per-sequence W_down0,
    look-ahead rows, a ragged last chunk."""
    for seed, pad, per_seq, la in ((33, "sequence", False, 1), (34, "chunk", True, 0),
                                   (35, "chunk", False, 2)):
        x = backward_case(seed, per_seq=per_seq, lookahead=la, T=30, C=8)
        g = backward(x, pad=pad)
        t = {k: torch.tensor(np.asarray(x[k], np.float64), requires_grad=True)
             for k in BWD_KEYS}
        O, Wf = _torch_prefill(t, x["eta"], x["chunk"], pad)
        loss = (O * torch.tensor(x["dO"])).sum() + (Wf * torch.tensor(x["dW_final"])).sum()
        loss.backward()
        for key in BWD_KEYS:
            _close(g[GRAD_OF[key]], t[key].grad.numpy(), tol=1e-10,
                   what=f"{GRAD_OF[key]} ({pad})")


def pin_backward_plain_mlp():
    """eta = 0: the layer is the plain gated MLP O = Z W_down0^T and W_final
    = W_down0, so the target path gets no gradient (dX0, dtaps, dW_target
    exactly zero), dW_down0 = sum over sequences of dO^T Z + dW_final, and
    dH, dW_g, dW_u are the plain MLP's (torch autograd of silu and matmul)."""
    x = backward_case(36, T=21, C=8)
    g = backward(x, eta=0.0)
    for key in ("dX0", "dtaps", "dW_target"):
        assert not np.any(g[key]), f"{key} must be zero at eta = 0"
    H = torch.tensor(x["H"], requires_grad=True)
    Wg = torch.tensor(x["Wg"], requires_grad=True)
    Wu = torch.tensor(x["Wu"], requires_grad=True)
    W0 = torch.tensor(x["W_down0"], requires_grad=True)
    Z = torch.nn.functional.silu(H @ Wg.T) * (H @ Wu.T)
    loss = ((Z @ W0.T) * torch.tensor(x["dO"])).sum() + (torch.tensor(x["dW_final"]).sum(0) * W0).sum()
    loss.backward()
    _close(g["dH"], H.grad.numpy(), what="plain dH")
    _close(g["dWg"], Wg.grad.numpy(), what="plain dWg")
    _close(g["dWu"], Wu.grad.numpy(), what="plain dWu")
    _close(g["dW_down0"], W0.grad.numpy(), what="plain dW_down0")


def pin_backward_linear_in_upstream():
    """The gradients are linear in (dO, dW_final) jointly."""
    x = backward_case(37, T=19, C=8)
    rng = np.random.default_rng(37)
    dO2, dW2 = rng.standard_normal(x["dO"].shape), rng.standard_normal(x["dW_final"].shape)
    g1 = backward(x)
    g2 = backward(x, dO=dO2, dW_final=dW2)
    g3 = backward(x, dO=x["dO"] - 3.0 * dO2, dW_final=x["dW_final"] - 3.0 * dW2)
    for key in GRAD_OF.values():
        _close(g3[key], g1[key] - 3.0 * g2[key], tol=1e-12, what=f"linear {key}")


ALL_PINS = [pin_reduces_to_plain_mlp, pin_prefix_scan_form, pin_state_free_form,
            pin_next_token_target, pin_conv_library, pin_linear_in_eta,
            pin_chunk_causality, pin_batch_independence, pin_split_resume,
            pin_brute_force_scalars, pin_sampled_forms, pin_golden_ntp_fixture,
            pin_packed_single_document, pin_packed_equals_documents,
            pin_packed_isolation, pin_packed_clip_equals_documents, pin_clip_loose_is_plain, pin_clip_each_delta,
            pin_decode_is_chunk_padded_prefill, pin_decode_pending_chunk,
            pin_decode_resumes_prefill, pin_backward_finite_differences,
            pin_backward_autograd, pin_backward_plain_mlp, pin_backward_linear_in_upstream]
