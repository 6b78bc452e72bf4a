"""CPU-only: plant a plausible mistake in the oracle, rerun every pin, and
check that at least one pin catches it. This is what shows the pins are
strong enough to trust the oracle; every mutation lives here, on the CPU.
"""
import numpy as np
import pytest

import oracle.ttt_oracle as ora
import oracle_pins

_real_prefill = ora.ttt_prefill
_real_target = ora.lm_target
_real_conv = ora.conv_target_input


def _prefill_variant(order="apply_first", scale=1.0, skip_last=False,
                     shared_state=False, sign=1.0, chunk_extra=0, clip_mode="delta"):
    """A copy of the recurrence with one knob turned away from the pages.
    clip_mode: "delta" (the pages), "no_eta" (the norm of V^T Z without
    eta), "inverted" (scale norm / clip), "state" (clip the whole state)."""
    def prefill(H, X0, Wg, Wu, W_down0, taps, W_target, eta, chunk,
                pad="sequence", clip=None):
        H, X0, W_down0 = (np.asarray(a, np.float64) for a in (H, X0, W_down0))
        B, T, d = H.shape
        f = Wg.shape[0]
        O = np.zeros((B, T, d))
        Wf = np.zeros((B, d, f))
        W = None
        step = chunk + chunk_extra
        for b in range(B):
            Z = ora.gated_activation(H[b], Wg, Wu)
            V = ora.lm_target(X0[b], taps, W_target, pad, chunk, n_out=T)
            if W is None or not shared_state:
                W = (W_down0[b] if W_down0.ndim == 3 else W_down0).copy()
            starts = list(range(0, T, step))
            for n, s in enumerate(starts):
                r = slice(s, min(s + step, T))
                upd = sign * eta * scale * (V[r].T @ Z[r])
                if clip is not None:
                    if clip_mode == "delta":
                        nrm = np.linalg.norm(upd)
                        upd = upd * min(1.0, clip / nrm) if nrm > 0 else upd
                    elif clip_mode == "no_eta":
                        nrm = np.linalg.norm(V[r].T @ Z[r])
                        upd = upd * min(1.0, clip / nrm) if nrm > 0 else upd
                    elif clip_mode == "inverted":
                        nrm = np.linalg.norm(upd)
                        upd = upd * min(1.0, nrm / clip)
                if skip_last and n == len(starts) - 1:
                    upd = 0.0
                if order == "update_first":
                    W = W + upd
                    O[b, r] = Z[r] @ W.T
                else:
                    O[b, r] = Z[r] @ W.T
                    W = W + upd
                if clip is not None and clip_mode == "state":
                    nrm = np.linalg.norm(W)
                    W = W * min(1.0, clip / nrm)
            Wf[b] = W
        return O, Wf
    return prefill


def _target_transposed(X0, taps, W_target, pad="sequence", chunk=None, n_out=None):
    return _real_conv(X0, taps, pad, chunk, n_out) @ np.asarray(W_target, np.float64).T


def _conv_backward(X0, taps, pad="sequence", chunk=None, n_out=None):
    X0 = np.asarray(X0, np.float64)
    return _real_conv(X0[::-1], taps, pad, chunk, n_out)[::-1].copy()


def _conv_wraps(X0, taps, pad="sequence", chunk=None, n_out=None):
    X0 = np.asarray(X0, np.float64)
    T = X0.shape[0] if n_out is None else n_out
    Y = np.zeros((T, X0.shape[1]))
    for k in range(taps.shape[0]):
        Y += np.asarray(taps[k], np.float64) * np.roll(X0, -k, axis=0)[:T]
    return Y


def _conv_ignores_chunk(X0, taps, pad="sequence", chunk=None, n_out=None):
    return _real_conv(X0, taps, "sequence", chunk, n_out)


_real_packed = ora.ttt_prefill_packed


def _packed_variant(reset=True, conv_stops=True, chunks_from_doc=True, clips=True):
    """A copy of the packed recurrence with one knob turned away from the
    pages: no state reset at a document start, a conv that reads across the
    boundary, chunks counted from token 0 instead of the document start, or
    a clipping limit that is ignored."""
    def packed(H, X0, Wg, Wu, W_down0, taps, W_target, eta, chunk, doc_starts,
               pad="sequence", clip=None):
        H, X0, taps = (np.asarray(a, np.float64) for a in (H, X0, taps))
        W0 = np.asarray(W_down0, np.float64)
        T, d = H.shape
        starts = list(doc_starts)
        bounds = starts + [T]
        cuts = set()
        for a, e in zip(bounds, bounds[1:]):
            base = a if chunks_from_doc else 0
            cuts.update(c for c in range(base, e, chunk) if c >= a)
            cuts.add(a)
        cuts = sorted(cuts) + [T]
        doc_end = np.zeros(T, int)
        for a, e in zip(bounds, bounds[1:]):
            doc_end[a:e] = e
        chunk_end = np.zeros(T, int)
        for a, e in zip(cuts, cuts[1:]):
            chunk_end[a:e] = e
        lim = (doc_end if conv_stops else np.full(T, T)) if pad == "sequence" else chunk_end
        Y = np.zeros((T, d))
        for t in range(T):
            for k in range(taps.shape[0]):
                if t + k < lim[t]:
                    Y[t] += taps[k] * X0[t + k]
        V = Y @ np.asarray(W_target, np.float64)
        Z = ora.gated_activation(H, Wg, Wu)
        O = np.zeros((T, d))
        W = W0.copy()
        for a, e in zip(cuts, cuts[1:]):
            if reset and a in starts:
                W = W0.copy()
            O[a:e] = Z[a:e] @ W.T
            delta = eta * (V[a:e].T @ Z[a:e])
            norm = np.linalg.norm(delta)
            if clips and clip is not None and norm > clip:
                delta = delta * (clip / norm)
            W = W + delta
        return O, W
    return packed


_real_decode = ora.ttt_decode


def _decode_variant(late=0, update_first=False, conv_past_chunk=False):
    """A copy of the decode loop with one knob turned: the chunk's update
    taken `late` tokens after the chunk closes, taken before the closing
    token's output, or a chunk target that reads the next chunk's tokens."""
    def decode(H, X0, Wg, Wu, W_state, taps, W_target, eta, chunk, start=0):
        H, X0, taps = (np.asarray(a, np.float64) for a in (H, X0, taps))
        Ws = np.asarray(W_state, np.float64)
        B, n, d = H.shape
        f = np.asarray(Wg).shape[0]
        K = taps.shape[0]
        O = np.zeros((B, n, d))
        W_out = np.zeros((B, d, f))
        pend = 0
        for b in range(B):
            W = (Ws[b] if Ws.ndim == 3 else Ws).copy()
            Z = ora.gated_activation(H[b], Wg, Wu)
            queue = []                  # (token index when due, delta)
            c0 = 0
            for i in range(n):
                closes = (start + i + 1) % chunk == 0
                if closes and update_first:
                    pass
                for due, dl in [q for q in queue if q[0] <= i]:
                    W = W + dl
                queue = [q for q in queue if q[0] > i]
                rows = slice(c0, i + 1)
                if closes:
                    L = i + 1 - c0
                    lim = min(n, c0 + L + K - 1) if conv_past_chunk else c0 + L
                    Y = np.zeros((L, d))
                    for t in range(L):
                        for k in range(K):
                            if c0 + t + k < lim:
                                Y[t] += taps[k] * X0[b, c0 + t + k]
                    dl = eta * ((Y @ np.asarray(W_target, np.float64)).T @ Z[rows])
                    if update_first:
                        W = W + dl
                        O[b, i] = W @ Z[i]
                    else:
                        O[b, i] = W @ Z[i]
                        if late == 0:
                            W = W + dl
                        else:
                            queue.append((i + 1 + late, dl))
                    c0 = i + 1
                else:
                    O[b, i] = W @ Z[i]
            for _, dl in queue:
                W = W + dl
            W_out[b] = W
            pend = n - c0
        return O, W_out, pend
    return decode


def _backward_variant(mistake):
    """A copy of the backward with one plausible mistake planted: the apply's
    gradient taken against the state after the chunk's update ("next_state"),
    the update's term of dZ dropped ("no_update_term"), the chunk's own
    apply folded into the state gradient before its update terms
    ("inclusive_gbar"), dW_final ignored ("no_dw_final"), phi' taken as
    sigma ("silu_prime"), dW_target transposed ("dwt_transposed"), the
    conv's input gradient scattered backwards ("conv_backwards"), eta left
    out of dV ("dv_no_eta")."""
    def bwd(H, X0, Wg, Wu, W_down0, taps, W_target, eta, chunk, dO, dW_final=None,
            pad="sequence"):
        H, X0, W_down0 = (np.asarray(a, np.float64) for a in (H, X0, W_down0))
        Wg, Wu, taps, Wt, dO = (np.asarray(a, np.float64) for a in (Wg, Wu, taps, W_target, dO))
        B, T, d = H.shape
        f, K, T_in = Wg.shape[0], taps.shape[0], X0.shape[1]
        dWf = np.zeros((B, d, f)) if dW_final is None or mistake == "no_dw_final" \
            else np.asarray(dW_final, np.float64)
        out = {"dH": np.zeros((B, T, d)), "dX0": np.zeros_like(X0), "dWg": np.zeros((f, d)),
               "dWu": np.zeros((f, d)), "dW_down0": np.zeros_like(W_down0),
               "dtaps": np.zeros((K, d)), "dW_target": np.zeros((d, d))}
        ti = np.arange(T)
        bound = np.full(T, T_in) if pad == "sequence" else np.minimum((ti // chunk + 1) * chunk, T_in)
        starts = list(range(0, T, chunk))
        for b in range(B):
            G, U = H[b] @ Wg.T, H[b] @ Wu.T
            sig = 1.0 / (1.0 + np.exp(-G))
            S = G * sig
            Z = S * U
            Y = _real_conv(X0[b], taps, pad, chunk, n_out=T)
            V = Y @ Wt
            W = (W_down0[b] if W_down0.ndim == 3 else W_down0).copy()
            states = []
            for a in starts:
                states.append(W)
                W = W + eta * (V[a:a + chunk].T @ Z[a:a + chunk])
            states.append(W)
            Gbar = dWf[b].copy()
            dZ, dV = np.zeros((T, f)), np.zeros((T, d))
            for i in reversed(range(len(starts))):
                r = slice(starts[i], min(starts[i] + chunk, T))
                if mistake == "inclusive_gbar":
                    Gbar = Gbar + dO[b, r].T @ Z[r]
                dV[r] = (1.0 if mistake == "dv_no_eta" else eta) * (Z[r] @ Gbar.T)
                upd = 0.0 if mistake == "no_update_term" else eta * (V[r] @ Gbar)
                dZ[r] = upd + dO[b, r] @ states[i + 1 if mistake == "next_state" else i]
                if mistake != "inclusive_gbar":
                    Gbar = Gbar + dO[b, r].T @ Z[r]
            if W_down0.ndim == 3:
                out["dW_down0"][b] = Gbar
            else:
                out["dW_down0"] += Gbar
            dY = dV @ Wt.T
            out["dW_target"] += (dV.T @ Y) if mistake == "dwt_transposed" else (Y.T @ dV)
            for k in range(K):
                m = ti + k < bound
                tt = ti[m]
                out["dtaps"][k] += (dY[tt] * X0[b, tt + k]).sum(axis=0)
                dst = np.clip(tt - k, 0, T_in - 1) if mistake == "conv_backwards" else tt + k
                out["dX0"][b, dst] += taps[k] * dY[tt]
            dphi = sig if mistake == "silu_prime" else sig * (1.0 + G * (1.0 - sig))
            dG, dU = dZ * U * dphi, dZ * S
            out["dH"][b] = dG @ Wg + dU @ Wu
            out["dWg"] += dG.T @ H[b]
            out["dWu"] += dU.T @ H[b]
        return out
    return bwd


MUTATIONS = {
    **{f"backward_{m}": ("ttt_prefill_backward", _backward_variant(m))
       for m in ("next_state", "no_update_term", "inclusive_gbar", "no_dw_final", "silu_prime",
                 "dwt_transposed", "conv_backwards", "dv_no_eta")},
    "decode_update_one_token_late": ("ttt_decode", _decode_variant(late=1)),
    "decode_update_before_last_output": ("ttt_decode", _decode_variant(update_first=True)),
    "decode_target_reads_next_chunk": ("ttt_decode", _decode_variant(conv_past_chunk=True)),
    "clip_norm_without_eta": ("ttt_prefill", _prefill_variant(clip_mode="no_eta")),
    "clip_scale_inverted": ("ttt_prefill", _prefill_variant(clip_mode="inverted")),
    "clip_whole_state": ("ttt_prefill", _prefill_variant(clip_mode="state")),
    "packed_no_reset": ("ttt_prefill_packed", _packed_variant(reset=False)),
    "packed_conv_crosses_documents": ("ttt_prefill_packed", _packed_variant(conv_stops=False)),
    "packed_chunks_from_token_0": ("ttt_prefill_packed", _packed_variant(chunks_from_doc=False)),
    "packed_clip_ignored": ("ttt_prefill_packed", _packed_variant(clips=False)),
    "inclusive_prefix_leak": ("ttt_prefill", _prefill_variant(order="update_first")),
    "skip_update": ("ttt_prefill", _prefill_variant(scale=0.0)),
    "normalise_by_chunk": ("ttt_prefill", _prefill_variant(scale=1.0 / 8)),
    "wrong_sign": ("ttt_prefill", _prefill_variant(sign=-1.0)),
    "drop_last_update": ("ttt_prefill", _prefill_variant(skip_last=True)),
    "state_shared_across_batch": ("ttt_prefill", _prefill_variant(shared_state=True)),
    "chunk_off_by_one": ("ttt_prefill", _prefill_variant(chunk_extra=1)),
    "w_target_transposed": ("lm_target", _target_transposed),
    "conv_reads_backward": ("conv_target_input", _conv_backward),
    "conv_wraps_around": ("conv_target_input", _conv_wraps),
    "chunk_padding_ignored": ("conv_target_input", _conv_ignores_chunk),
    "phi_is_sigmoid": ("silu", lambda x: 1.0 / (1.0 + np.exp(-x))),
    "phi_is_identity": ("silu", lambda x: x),
    "gate_up_swapped": ("gated_activation",
                        lambda H, Wg, Wu: ora.silu(np.asarray(H, np.float64) @ np.asarray(Wu, np.float64).T)
                        * (np.asarray(H, np.float64) @ np.asarray(Wg, np.float64).T)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ora, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutation {name} passed every pin"
