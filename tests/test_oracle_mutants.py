"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutant patches one step of oracle.ttt_oracle for the duration of a test:
a plausible slip (a dropped term, a wrong sign, shift or index, a transposed
operand, an off-by-one chunk). The pins must catch every one of them.
"""
import numpy as np
import pytest

import oracle
import oracle.ttt_oracle as ot
from tests import pins


def _loop_mutant(kind):
    def one(x, ids, E_tgt, W_up, W_gate, W_entry, C, eta, clip_tau=None, conv_w=None, W_target=None):
        x = np.asarray(x, dtype=np.float64)
        T = x.shape[0]
        S = np.asarray(W_entry, dtype=np.float64).copy()
        y = np.zeros((T, S.shape[0]))
        if T == 0:
            return y, S
        Z = ot.gated_activation(x, W_up, W_gate)
        V = ot.ntp_targets(ids, E_tgt) if conv_w is None else ot.conv_targets(ids, E_tgt, conv_w, W_target, C)
        S0 = S.copy()
        ranges = ot.chunk_ranges(T, C)
        for n, (s, e) in enumerate(ranges):
            dW = ot.clip_update(eta * (V[s:e].T @ Z[s:e]), clip_tau)
            if kind == "clip_accumulated":
                # clips the change accumulated since the entry state, not the chunk update
                y[s:e] = Z[s:e] @ S.T
                S = S0 + ot.clip_update(S - S0 + eta * (V[s:e].T @ Z[s:e]), clip_tau)
                continue
            if kind == "clip_before_eta" and clip_tau is not None:
                raw = V[s:e].T @ Z[s:e]
                n = np.linalg.norm(raw)
                dW = eta * raw * (min(1.0, clip_tau / n) if n > 0 else 1.0)
            if kind == "update_then_apply":
                S = S + dW
                y[s:e] = Z[s:e] @ S.T
                continue
            if kind == "transposed_apply":
                y[s:e] = Z[s:e] @ S  # only shape-valid when d == f
            else:
                y[s:e] = Z[s:e] @ S.T
            if kind == "sign":
                S = S - dW
            elif kind == "mean":
                S = S + dW / (e - s)
            elif kind == "no_carry":
                S = S0 + dW
            elif kind == "no_eta":
                S = S + dW / eta if eta != 0 else S
            elif kind == "drop_last_update" and n == len(ranges) - 1:
                pass
            elif kind == "transposed_update":
                S = S + eta * (Z[s:e].T @ V[s:e]).T.T if S.shape[0] == S.shape[1] else S + dW
            else:
                S = S + dW
        return y, S
    return one


def _targets_shift(k):
    def ntp(ids, E_tgt):
        ids = np.asarray(ids)
        E = np.asarray(E_tgt, dtype=np.float64)
        T = ids.shape[0] - 1
        V = np.zeros((T, E.shape[1]))
        for t in range(T):
            j = t + k
            if 0 <= j <= T and 0 <= ids[j] < E.shape[0]:
                V[t] = E[ids[j]]
        return V
    return ntp


def _targets_clip(ids, E_tgt):
    ids = np.asarray(ids)
    E = np.asarray(E_tgt, dtype=np.float64)
    nxt = np.clip(ids[1:], 0, E.shape[0] - 1)
    return E[nxt]


def _gate_on_up(x, W_up, W_gate):
    x = np.asarray(x, dtype=np.float64)
    return ot.silu(x @ np.asarray(W_up).T) * (x @ np.asarray(W_gate).T)


def _no_silu(x, W_up, W_gate):
    x = np.asarray(x, dtype=np.float64)
    return (x @ np.asarray(W_gate).T) * (x @ np.asarray(W_up).T)


def _chunks_plus_one(T, C):
    return [(s, min(s + C + 1, T)) for s in range(0, T, C + 1)]


def _chunks_overlap(T, C):
    return [(max(0, s - 1), min(s + C, T)) for s in range(0, T, C)]


def _clip_always(dW, tau):
    # rescales every update to norm tau (a normalisation, not a clip)
    return dW if tau is None else dW * (tau / np.linalg.norm(dW))


def _clip_maxabs(dW, tau):
    if tau is None:
        return dW
    n = np.max(np.abs(dW))
    return dW * (tau / n) if n > tau else dW


def _clip_spectral(dW, tau):
    if tau is None:
        return dW
    n = np.linalg.norm(dW, 2)
    return dW * (tau / n) if n > tau else dW


def _clip_squared(dW, tau):
    if tau is None:
        return dW
    n2 = float(np.sum(dW * dW))
    return dW * (tau / n2) if n2 > tau else dW


def _conv_mutant(kind):
    def conv(ids, E_in, conv_w, W_target, C):
        ids = np.asarray(ids)
        E = np.asarray(E_in, dtype=np.float64)
        cw = np.asarray(conv_w, dtype=np.float64)
        T = ids.shape[0] - 1
        U = np.zeros((T, E.shape[1]))
        for t in range(T):
            limit = min((t // C + 1) * C, T)
            if kind == "no_padding":
                limit = T
            elif kind == "strict_padding":
                limit = min((t // C + 1) * C - 1, T)
            for k in range(cw.shape[0]):
                p = t + k if kind == "offset_0" else t + 1 + k
                if p > limit:
                    break
                tok = int(ids[p])
                if 0 <= tok < E.shape[0]:
                    U[t] += (cw[cw.shape[0] - 1 - k] if kind == "reversed_taps" else cw[k]) * E[tok]
        Wt = np.asarray(W_target, dtype=np.float64)
        return U @ (Wt.T if kind == "transposed_W_target" else Wt)
    return conv


def _docs_mutant(kind):
    def docs(x, ids, E_tgt, W_up, W_gate, W_entry, W_reset, C, eta, doc_starts, clip_tau=None, conv_w=None,
             W_target=None):
        x = np.asarray(x, dtype=np.float64)
        B, T = x.shape[0], x.shape[1]
        W_entry = np.asarray(W_entry, dtype=np.float64)
        ys, Ws = [], []
        for b in range(B):
            S = (W_entry if W_entry.ndim == 2 else W_entry[b]).copy()
            starts = [r + 1 if kind == "late_reset" else r for r in doc_starts[b]]
            bounds = [0] + starts + [T]
            yb = np.zeros((T, S.shape[0]))
            for j in range(len(bounds) - 1):
                s0, s1 = bounds[j], bounds[j + 1]
                if j > 0 and kind != "no_reset":
                    S = (W_entry if kind == "reset_to_entry" else np.asarray(W_reset, dtype=np.float64)).copy()
                ids_seg = np.array(ids[b][s0:s1 + 1], copy=True)
                if j < len(bounds) - 2 and kind != "lookahead_kept":
                    ids_seg[-1] = -1
                yb[s0:s1], S = ot.ttt_forward_one(x[b, s0:s1], ids_seg, E_tgt, W_up, W_gate, S, C, eta,
                                                  clip_tau, conv_w, W_target)
            ys.append(yb)
            Ws.append(S)
        return np.stack(ys), np.stack(Ws)
    return docs


def _sigmoid_wrong(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(g))


MUTANTS = {
    "target_shift_0 (reconstruction)": ("ntp_targets", _targets_shift(0)),
    "target_shift_2": ("ntp_targets", _targets_shift(2)),
    "targets_clip_ids": ("ntp_targets", _targets_clip),
    "silu_on_up_path": ("gated_activation", _gate_on_up),
    "no_silu": ("gated_activation", _no_silu),
    "silu_sign": ("silu", _sigmoid_wrong),
    "chunks_of_C_plus_1": ("chunk_ranges", _chunks_plus_one),
    "chunks_overlap": ("chunk_ranges", _chunks_overlap),
    "update_then_apply": ("ttt_forward_one", _loop_mutant("update_then_apply")),
    "update_sign": ("ttt_forward_one", _loop_mutant("sign")),
    "update_mean": ("ttt_forward_one", _loop_mutant("mean")),
    "no_state_carry": ("ttt_forward_one", _loop_mutant("no_carry")),
    "no_eta": ("ttt_forward_one", _loop_mutant("no_eta")),
    "drop_last_update": ("ttt_forward_one", _loop_mutant("drop_last_update")),
    "transposed_apply": ("ttt_forward_one", _loop_mutant("transposed_apply")),
    "clip_always_to_tau": ("clip_update", _clip_always),
    "clip_max_abs_norm": ("clip_update", _clip_maxabs),
    "clip_spectral_norm": ("clip_update", _clip_spectral),
    "clip_squared_norm": ("clip_update", _clip_squared),
    "clip_accumulated_change": ("ttt_forward_one", _loop_mutant("clip_accumulated")),
    "clip_before_eta": ("ttt_forward_one", _loop_mutant("clip_before_eta")),
    "conv_taps_from_current_token": ("conv_targets", _conv_mutant("offset_0")),
    "conv_no_chunk_padding": ("conv_targets", _conv_mutant("no_padding")),
    "conv_no_crossing_at_all": ("conv_targets", _conv_mutant("strict_padding")),
    "conv_reversed_taps": ("conv_targets", _conv_mutant("reversed_taps")),
    "conv_transposed_W_target": ("conv_targets", _conv_mutant("transposed_W_target")),
    "docs_no_reset": ("ttt_forward_docs", _docs_mutant("no_reset")),
    "docs_reset_to_carried_state": ("ttt_forward_docs", _docs_mutant("reset_to_entry")),
    "docs_reset_one_token_late": ("ttt_forward_docs", _docs_mutant("late_reset")),
}


def _run_pins(fwd):
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(fwd)
        except (AssertionError, ValueError, IndexError) as e:
            failures.append(str(e)[:80])
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, repl = MUTANTS[name]
    monkeypatch.setattr(ot, attr, repl)
    with np.errstate(invalid="ignore", divide="ignore"):  # some planted mistakes divide by a zero norm
        failures = _run_pins(ot.ttt_forward)
    assert failures, f"planted mistake '{name}' passed every pin"


def test_unmutated_oracle_passes_all_pins():
    assert _run_pins(oracle.ttt_forward) == []
