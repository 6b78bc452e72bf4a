"""CPU oracle for the In-Place TTT fast-weight gated-MLP prefill.

TEST INFRASTRUCTURE ONLY. This is a plain, slow, float64 NumPy statement of
what the layer computes. Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import or call it; the HIP library never
does, and shares no code with it.

Sources (page title, then section / equation):
  [notes]  "论文精读：In-Place Test-Time Training" reading notes (jindou-blog):
           "In-Place 设计" gated-MLP equation; "Chunk-Wise 更新机制" update
           equation; "LM-Aligned 目标函数" target equation.
  [forum]  "In-Place TTT: ByteDance Seed's Test-Time Training Framework Gives
           LLMs On-the-Fly Memory" (zhichai): "Three Core Designs" 1-3.
  [iplex]  iplexlaw explainer of "In-Place Test-Time Training": §2 (W_down as
           fast weight), §3 (apply, then update), §4 (LM-aligned target),
           §6 (prefix scan, chunk-boundary padding, document reset).

Readings where the pages leave a step open (each is a choice, stated here and
tested by the pins in tests/test_oracle.py):
  * phi is SiLU, x * sigmoid(x).
  * Tap k of the depthwise conv reads X0[t + k]; so taps [0, 1, 0, ...] with
    W_target = I give the next token's embedding ([forum] design 3). Rows past
    the end of the sequence are zero ("sequence" padding). The [iplex] §6
    remark that the conv must not pull information across chunk boundaries
    is the optional "chunk" padding: reads stop at the end of the token's own
    chunk.
  * V = conv(X0) @ W_target, W_target[i, j] maps input channel i to output
    channel j (right multiplication, no transpose).
  * W_down is [d, f]; the output is O = Z W_down^T and the update is
    W += eta * V_i^T Z_i, with no 1/C factor and no clipping.
  * Each sequence of the batch has its own state, starting from W_down0.
  * A last chunk shorter than C is allowed. The returned final state includes
    the last chunk's update.
  * Update-norm clipping ([iplex] §6, §8: the Frobenius norm of the update
    delta is limited to a threshold): optionally, each chunk's delta
    eta * V_i^T Z_i is scaled by min(1, clip / ||eta * V_i^T Z_i||_F). The
    threshold the pages print (1e-5) reads as garbled, so it is a parameter;
    clip = None (the default) applies no clipping.
  * Packed documents ([iplex] §6, document boundaries): a sequence may hold
    several documents back to back, given by their start offsets. At each
    document start the state returns to W_down0 and the chunking restarts,
    and the conv reads nothing past the token's own document (nor past its
    chunk, with chunk padding). Clipping, when asked for, acts on each chunk
    of each document. The returned final state is the one after the last
    document.
  * Decode (ttt_decode): one token at a time, with chunk-local conv padding
    only, the state stepped as soon as a chunk's last token is processed.
    With that padding it is the prefill computed token by token; the pages
    say decode was not evaluated and give no rule for sequence padding.
  * Backward (ttt_prefill_backward): the pages train the layer's slow
    parameters by continual pretraining ([iplex] §2 and §7.1; [forum]
    "Limitations"), and the conv taps and W_target reach the output only
    through the fast-weight updates ([iplex] §6 initialises them so that the
    first updates are near zero). So the backward is the exact gradient of
    the prefill, taken through the chunk recurrence, with respect to every
    input: H, X0, W_g, W_u, W_down0, the taps and W_target. eta is a fixed
    scalar (the pages do not learn it) and gets no gradient.
"""
from __future__ import annotations

import numpy as np

__all__ = ["silu", "gated_activation", "conv_target_input", "lm_target",
           "ttt_prefill", "ttt_prefill_packed", "ttt_decode", "ttt_prefill_backward",
           "activation_rows", "target_rows", "final_state_entries"]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    """phi(x) = x * sigmoid(x) = x / (1 + exp(-x))."""
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def gated_activation(H, Wg, Wu) -> np.ndarray:
    """Z = phi(H Wg^T) * (H Wu^T), elementwise product.

    [notes] "In-Place 设计": the gated MLP's intermediate activation, the part
    of O = (phi(H W_gate^T) . (H W_up^T)) W_down^T that stays frozen; [iplex] §2.
    H [T, d], Wg and Wu [f, d] -> Z [T, f].
    """
    H, Wg, Wu = _f64(H), _f64(Wg), _f64(Wu)
    return silu(H @ Wg.T) * (H @ Wu.T)


def conv_target_input(X0, taps, pad="sequence", chunk=None, n_out=None):
    """Depthwise conv of the token embeddings, the Conv1D(X0) of the target.

    [notes] "LM-Aligned 目标函数" target equation; [iplex] §4, §6 (depthwise).
    Y[t, c] = sum_k taps[k, c] * X0[t + k, c], where the read X0[t + k]
    counts only if t + k is inside the sequence (pad="sequence") or inside
    t's own chunk of `chunk` tokens (pad="chunk"). X0 may carry extra
    look-ahead rows past the n_out outputs wanted.
    """
    X0, taps = _f64(X0), _f64(taps)
    T_in, d = X0.shape
    T = T_in if n_out is None else n_out
    K = taps.shape[0]
    Y = np.zeros((T, d))
    for k in range(K):
        if pad == "sequence":
            # output t reads row t + k while t + k < T_in
            hi = min(T, T_in - k)
            if hi > 0:
                Y[:hi] += taps[k] * X0[k:hi + k]
        elif pad == "chunk":
            # output t in chunk [a, a + chunk) reads row t + k while it is in
            # that chunk (and inside X0)
            for a in range(0, T, chunk):
                hi = min(a + chunk, T, min(a + chunk, T_in) - k)
                if hi > a:
                    Y[a:hi] += taps[k] * X0[a + k:hi + k]
        else:
            raise ValueError(pad)
    return Y


def lm_target(X0, taps, W_target, pad="sequence", chunk=None, n_out=None):
    """V = Conv1D(X0) W_target, the LM-aligned target ([notes] target
    equation; [forum] design 3; [iplex] §4)."""
    return conv_target_input(X0, taps, pad, chunk, n_out) @ _f64(W_target)


def ttt_prefill(H, X0, Wg, Wu, W_down0, taps, W_target, eta, chunk,
                pad="sequence", clip=None):
    """The layer's prefill: per-chunk apply, then update, over the sequence.

    [notes] "Chunk-Wise 更新机制": the sequence is cut into non-overlapping
    chunks; each chunk first produces its output with the current fast
    weight, then the fast weight takes the step
    W^(i+1) = W^(i) + eta * V_[i]^T Z_[i]. [iplex] §3: a chunk's output always
    uses the state from before its own update. [iplex] §6: the state starts
    at the pretrained W_down for each document (here: each batch row).

    H [B, T, d]; X0 [B, T + L, d] (L >= 0 look-ahead rows, read by the conv
    only); Wg, Wu [f, d]; W_down0 [d, f] shared, or [B, d, f] per sequence;
    taps [K, d]; W_target [d, d]. Returns O [B, T, d] and the final state
    W [B, d, f], float64. clip: None, or the Frobenius-norm limit of each
    chunk's update delta ([iplex] §6 norm clipping).
    """
    H, X0, W_down0 = _f64(H), _f64(X0), _f64(W_down0)
    B, T, d = H.shape
    f = Wg.shape[0]
    if X0.shape[0] != B or X0.shape[1] < T or X0.shape[2] != d:
        raise ValueError("X0 must be [B, >=T, d]")
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    O = np.zeros((B, T, d))
    W_final = np.zeros((B, d, f))
    for b in range(B):
        Z = gated_activation(H[b], Wg, Wu)                       # [T, f]
        V = lm_target(X0[b], taps, W_target, pad, chunk, n_out=T)  # [T, d]
        W = (W_down0[b] if W_down0.ndim == 3 else W_down0).copy()
        for start in range(0, T, chunk):
            rows = slice(start, min(start + chunk, T))
            O[b, rows] = Z[rows] @ W.T                 # apply: pre-update state
            delta = eta * (V[rows].T @ Z[rows])
            if clip is not None:
                norm = np.linalg.norm(delta)           # Frobenius norm of the delta
                if norm > clip:
                    delta = delta * (clip / norm)
            W = W + delta                              # then update
        W_final[b] = W
    return O, W_final


def ttt_prefill_packed(H, X0, Wg, Wu, W_down0, taps, W_target, eta, chunk,
                       doc_starts, pad="sequence", clip=None):
    """Prefill of one packed sequence holding several documents.

    [iplex] §6: the fast weight is reset to the pretrained W_down at every
    document boundary, so documents do not leak into each other; the conv
    target stops at the boundary as it does at the end of a sequence.
    Written token by token over the packed sequence: each token is assigned
    its document r (doc_starts[r] <= t < doc_starts[r + 1], the last one
    running to T) and its chunk, counted from the document's start; the
    state is set to W_down0 when a document begins and stepped at the end of
    each chunk.

    H [T, d]; X0 [T, d]; Wg, Wu [f, d]; W_down0 [d, f]; taps [K, d];
    W_target [d, d]; doc_starts: increasing offsets, the first 0. clip: None,
    or the Frobenius-norm limit of each chunk's update delta, as in
    ttt_prefill ([iplex] §6 norm clipping; a chunk here never spans two
    documents). Returns O [T, d] and the state after the last document
    [d, f], float64.
    """
    H, X0, taps = _f64(H), _f64(X0), _f64(taps)
    W0, Wt = _f64(W_down0), _f64(W_target)
    T, d = H.shape
    K = taps.shape[0]
    starts = [int(s) for s in doc_starts]
    if not starts or starts[0] != 0 or any(b <= a for a, b in zip(starts, starts[1:])) \
            or starts[-1] >= T:
        raise ValueError("doc_starts must increase from 0 and stay below T")
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    bounds = starts + [T]
    doc_end = np.zeros(T, dtype=np.int64)     # first token after t's document
    chunk_end = np.zeros(T, dtype=np.int64)   # first token after t's chunk
    chunk_id = np.zeros(T, dtype=np.int64)    # running chunk index over documents
    n_chunks = 0
    for r in range(len(starts)):
        a, e = bounds[r], bounds[r + 1]
        for t in range(a, e):
            c = (t - a) // chunk
            doc_end[t] = e
            chunk_end[t] = min(e, a + (c + 1) * chunk)
            chunk_id[t] = n_chunks + c
        n_chunks += -(-(e - a) // chunk)
    # Target: Y[t] = sum_k taps[k] * X0[t + k] over reads before the bound.
    limit = doc_end if pad == "sequence" else chunk_end
    if pad not in ("sequence", "chunk"):
        raise ValueError(pad)
    Y = np.zeros((T, d))
    for t in range(T):
        for k in range(K):
            if t + k < limit[t]:
                Y[t] += taps[k] * X0[t + k]
    V = Y @ Wt
    Z = gated_activation(H, Wg, Wu)
    O = np.zeros((T, d))
    W = W0.copy()
    t = 0
    while t < T:
        if t in starts:
            W = W0.copy()                       # document start: reset
        rows = slice(t, int(chunk_end[t]))
        O[rows] = Z[rows] @ W.T                 # apply with the pre-update state
        delta = eta * (V[rows].T @ Z[rows])
        if clip is not None:
            norm = np.linalg.norm(delta)        # Frobenius norm of the delta
            if norm > clip:
                delta = delta * (clip / norm)
        W = W + delta                           # then update
        t = int(chunk_end[t])
    assert n_chunks == int(chunk_id[-1]) + 1
    return O, W


def ttt_decode(H, X0, Wg, Wu, W_state, taps, W_target, eta, chunk, start=0):
    """Token-by-token decode of B sequences, with chunk-local conv padding.

    [iplex] §3 and §6: within a chunk every output uses the state from before
    the chunk's update, and the chunk's update is taken once the chunk is
    complete; with the [iplex] §6 chunk-boundary padding the target of a
    chunk reads only that chunk's tokens, so the update needs no token past
    the chunk's end and a decoder can take it as soon as the chunk's last
    token has been processed. (With sequence padding the last K - 1 targets
    of a chunk read tokens that are not decoded yet; the pages give no rule
    for that case, so it is not defined here.)

    Processes tokens one at a time: token i of the call is document position
    start + i (start counts tokens already processed, chunks being counted
    from the document start). For each token: z = phi(h Wg^T) * (h Wu^T) and
    o = z W^T with the current state; (z, x0) join the current chunk; when
    the position closes a chunk, its target Y[t] = sum_k taps[k] X0[t + k]
    over reads inside the chunk, V = Y W_target, and W += eta V^T Z.

    H, X0 [B, n, d]; W_state [d, f] (shared start) or [B, d, f]; returns
    O [B, n, d], the state [B, d, f] after the last complete chunk, and the
    number of tokens of the incomplete chunk left pending (not yet applied to
    the state), all float64. `start` must be a multiple of `chunk` (a call
    begins at a chunk boundary).
    """
    H, X0, taps = _f64(H), _f64(X0), _f64(taps)
    Wg, Wu, Wt = _f64(Wg), _f64(Wu), _f64(W_target)
    Ws = _f64(W_state)
    B, n, d = H.shape
    f = Wg.shape[0]
    K = taps.shape[0]
    if chunk < 1 or start % chunk != 0:
        raise ValueError("start must be a multiple of chunk")
    O = np.zeros((B, n, d))
    W_out = np.zeros((B, d, f))
    pending = 0
    for b in range(B):
        W = (Ws[b] if Ws.ndim == 3 else Ws).copy()
        zs, xs = [], []
        for i in range(n):
            h = H[b, i]
            z = silu(Wg @ h) * (Wu @ h)                 # [f]
            O[b, i] = W @ z                             # o = z W^T, pre-update state
            zs.append(z)
            xs.append(X0[b, i])
            if (start + i + 1) % chunk == 0:            # the chunk is complete
                L = len(zs)
                Y = np.zeros((L, d))
                for t in range(L):
                    for k in range(K):
                        if t + k < L:                   # reads stay inside the chunk
                            Y[t] += taps[k] * xs[t + k]
                V = Y @ Wt
                W = W + eta * (V.T @ np.array(zs))
                zs, xs = [], []
        W_out[b] = W
        pending = len(zs)
    return O, W_out, pending


def ttt_prefill_backward(H, X0, Wg, Wu, W_down0, taps, W_target, eta, chunk, dO,
                         dW_final=None, pad="sequence"):
    """Gradients of the prefill: for L = <dO, O> + <dW_final, W_final> (the
    upstream gradients of ttt_prefill's two outputs, dW_final zero if None),
    the gradient of L with respect to every input of ttt_prefill.

    The forward, per sequence ([notes] "In-Place 设计", "Chunk-Wise 更新机制",
    "LM-Aligned 目标函数"; [iplex] §3): G = H Wg^T, U = H Wu^T, Z = phi(G) * U;
    Y = conv(X0), V = Y W_target; W_0 = W_down0; for chunk i,
    O_i = Z_i W_i^T, then W_{i+1} = W_i + eta V_i^T Z_i; W_final = W_k.

    Reverse, chunk by chunk from the last: with Gbar = dL/dW_{i+1} (Gbar =
    dW_final after the last chunk),
        the update W_{i+1} = W_i + eta V_i^T Z_i gives
            dV_i += eta Z_i Gbar^T,   dZ_i += eta V_i Gbar;
        the apply O_i = Z_i W_i^T gives
            dZ_i += dO_i W_i,         dL/dW_i = Gbar + dO_i^T Z_i;
    and dW_down0 = dL/dW_0. Then V = Y W_target gives dY = dV W_target^T and
    dW_target = Y^T dV; the conv Y[t] = sum_k taps[k] X0[t + k] (reads before
    t's bound) gives dtaps[k] = sum_t dY[t] X0[t + k] and dX0[t + k] +=
    taps[k] dY[t] over the same reads; Z = phi(G) U with phi(x) = x sigma(x),
    phi'(x) = sigma(x) (1 + x (1 - sigma(x))), gives dG = dZ U phi'(G),
    dU = dZ phi(G), dH = dG Wg + dU Wu, dWg = dG^T H, dWu = dU^T H.

    Shapes as ttt_prefill (X0 may carry look-ahead rows past T; its gradient
    has X0's shape). dO [B, T, d]; dW_final None or [B, d, f]. Returns a dict
    of float64 arrays: dH, dX0, dWg, dWu, dW_down0 (the shape of W_down0:
    summed over the batch when it is shared), dtaps, dW_target.
    """
    H, X0, W_down0 = _f64(H), _f64(X0), _f64(W_down0)
    Wg, Wu, taps, Wt, dO = _f64(Wg), _f64(Wu), _f64(taps), _f64(W_target), _f64(dO)
    B, T, d = H.shape
    f = Wg.shape[0]
    K = taps.shape[0]
    T_in = X0.shape[1]
    if dO.shape != (B, T, d):
        raise ValueError("dO must be [B, T, d]")
    dWf = np.zeros((B, d, f)) if dW_final is None else _f64(dW_final)
    out = {"dH": np.zeros((B, T, d)), "dX0": np.zeros_like(X0), "dWg": np.zeros((f, d)),
           "dWu": np.zeros((f, d)), "dW_down0": np.zeros_like(W_down0),
           "dtaps": np.zeros((K, d)), "dW_target": np.zeros((d, d))}
    # the conv's read bound of each output t (as conv_target_input)
    t_idx = np.arange(T)
    if pad == "sequence":
        bound = np.full(T, T_in)
    elif pad == "chunk":
        bound = np.minimum((t_idx // chunk + 1) * chunk, T_in)
    else:
        raise ValueError(pad)
    starts = list(range(0, T, chunk))
    for b in range(B):
        G = H[b] @ Wg.T
        U = H[b] @ Wu.T
        sig = 1.0 / (1.0 + np.exp(-G))
        S = G * sig                                   # phi(G)
        Z = S * U
        Y = conv_target_input(X0[b], taps, pad, chunk, n_out=T)
        V = Y @ Wt
        # states before each chunk
        W = (W_down0[b] if W_down0.ndim == 3 else W_down0).copy()
        states = []
        for a in starts:
            r = slice(a, min(a + chunk, T))
            states.append(W)
            W = W + eta * (V[r].T @ Z[r])
        # reverse over the chunks
        Gbar = dWf[b].copy()
        dZ = np.zeros((T, f))
        dV = np.zeros((T, d))
        for i in reversed(range(len(starts))):
            r = slice(starts[i], min(starts[i] + chunk, T))
            dV[r] = eta * (Z[r] @ Gbar.T)
            dZ[r] = eta * (V[r] @ Gbar) + dO[b, r] @ states[i]
            Gbar = Gbar + dO[b, r].T @ Z[r]
        if W_down0.ndim == 3:
            out["dW_down0"][b] = Gbar
        else:
            out["dW_down0"] += Gbar
        dY = dV @ Wt.T
        out["dW_target"] += Y.T @ dV
        for k in range(K):
            m = t_idx + k < bound                      # the reads the forward made
            tt = t_idx[m]
            out["dtaps"][k] += (dY[tt] * X0[b, tt + k]).sum(axis=0)
            out["dX0"][b, tt + k] += taps[k] * dY[tt]
        dG = dZ * U * (sig * (1.0 + G * (1.0 - sig)))
        dU = dZ * S
        out["dH"][b] = dG @ Wg + dU @ Wu
        out["dWg"] += dG.T @ H[b]
        out["dWu"] += dU.T @ H[b]
    return out


# ---------------------------------------------------------------------------
# Sampled forms, for checking outputs of sizes the full recurrence is too slow
# for. Each is the same definition restricted to a few output elements.
# ---------------------------------------------------------------------------

def activation_rows(H_b, Wg, Wu, rows) -> np.ndarray:
    """Z[rows] of one sequence (the gated activation is row-local)."""
    return gated_activation(_f64(H_b)[rows], Wg, Wu)


def target_rows(X0_b, taps, W_target, rows, pad="sequence", chunk=None):
    """V[rows] of one sequence; each row reads X0 rows t..t+K-1 only."""
    X0_b, taps = _f64(X0_b), _f64(taps)
    T, d = X0_b.shape
    K = taps.shape[0]
    rows = np.asarray(rows)
    Y = np.zeros((len(rows), d))
    for i, t in enumerate(rows):
        end = T if pad == "sequence" else min(T, (t // chunk + 1) * chunk)
        for k in range(K):
            if t + k < end:
                Y[i] += taps[k] * X0_b[t + k]
    return Y @ _f64(W_target)


def final_state_entries(H_b, X0_b, Wg, Wu, W0_b, taps, W_target, eta, cs, js,
                        pad="sequence", chunk=None) -> np.ndarray:
    """Entries W_final[c, j] for c in cs, j in js of one sequence.

    Summing the update equation over all chunks gives
    W_final = W_down0 + eta * sum_i V_i^T Z_i = W_down0 + eta * V^T Z, since
    the chunks partition the tokens; each entry needs only column j of Z and
    column c of V over all tokens. X0_b may carry look-ahead rows past the
    T = len(H_b) tokens (read by the conv only).
    """
    H_b, Wg, Wu = _f64(H_b), _f64(Wg), _f64(Wu)
    cs, js = np.asarray(cs), np.asarray(js)
    Zc = silu(H_b @ Wg[js].T) * (H_b @ Wu[js].T)                  # [T, |js|]
    Y = conv_target_input(X0_b, taps, pad, chunk, n_out=H_b.shape[0])  # [T, d]
    Vc = Y @ _f64(W_target)[:, cs]                                  # [T, |cs|]
    return _f64(W0_b)[np.ix_(cs, js)] + eta * (Vc.T @ Zc)
