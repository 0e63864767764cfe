"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each check takes `fwd`, a callable with the signature of oracle.ttt_forward
(x [B][T][d], ids [B][T+1], E, W_up, W_gate, W_entry, C, eta, clip_tau=None)
-> (y, W_final),
and raises AssertionError when the callable disagrees with what the pages and
the mathematics fix. The planted-mistake tests run the same checks against
deliberately broken copies of the oracle and require each copy to fail one.

Independent references used here: torch.nn.functional.silu / embedding and
torch.autograd (fp64, CPU), a block-causal closed form, an explicit
parallel-prefix form, the per-token rule for C = 1, and invariants.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

RTOL = 1e-10


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def _close(a, b, tol=RTOL, what=""):
    r = _rel(a, b)
    assert r <= tol, f"{what}: max-rel {r:.3e} > {tol:.1e}"


def tiny_case(rng, d=6, f=10, B=1, T=12, vocab=9, w_scale=1.0):
    x = rng.standard_normal((B, T, d))
    Wu = rng.standard_normal((f, d)) / np.sqrt(d)
    Wg = rng.standard_normal((f, d)) / np.sqrt(d)
    W0 = w_scale * rng.standard_normal((d, f)) / np.sqrt(f)
    E = rng.standard_normal((vocab, d))
    ids = rng.integers(0, vocab, size=(B, T + 1)).astype(np.int32)
    return x, ids, E, Wu, Wg, W0


def _torch_z(x, Wu, Wg):
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    return (F.silu(xt @ torch.from_numpy(Wg).T) * (xt @ torch.from_numpy(Wu).T))


def _torch_v(ids_row, E):
    """Next-token rows by torch embedding; ids outside [0, vocab) give zero rows."""
    idx = torch.from_numpy(np.asarray(ids_row[1:], dtype=np.int64))
    Et = torch.from_numpy(np.asarray(E, dtype=np.float64))
    ok = (idx >= 0) & (idx < Et.shape[0])
    return F.embedding(torch.where(ok, idx, torch.zeros_like(idx)), Et) * ok[:, None].to(Et.dtype)


# P1: eta = 0 (any C) or C >= T (any eta, for y) reduces to the textbook gated MLP.
def check_static_mlp(fwd, seed=0, square=False):
    rng = np.random.default_rng(seed)
    d, f = (8, 8) if square else (6, 10)
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=d, f=f, B=2, T=13)
    y_ref = (_torch_z(x, Wu, Wg) @ torch.from_numpy(W0).T).numpy()
    for C in (1, 4, 13):
        y, W = fwd(x, ids, E, Wu, Wg, W0, C, 0.0)
        _close(y, y_ref, what=f"P1 eta=0 C={C} y")
        _close(W, np.broadcast_to(W0, W.shape), what=f"P1 eta=0 C={C} W_final")
    for C in (13, 20):
        y, _ = fwd(x, ids, E, Wu, Wg, W0, C, 0.37)
        _close(y, y_ref, what=f"P1 C>=T C={C} y")


# P2: one chunk (C = T): W_final = W0 - eta * grad L(W0) with L(W) = -sum_t <v_t, W z_t>.
def check_autograd_step(fwd, seed=1):
    rng = np.random.default_rng(seed)
    for (d, f, T) in ((4, 7, 5), (8, 16, 16), (5, 5, 3)):
        x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=d, f=f, B=1, T=T)
        eta = 0.173
        Z = _torch_z(x[0], Wu, Wg)
        V = _torch_v(ids[0], E)
        W = torch.from_numpy(W0.copy()).requires_grad_(True)
        loss = -(V * (Z @ W.T)).sum()
        loss.backward()
        W_ref = (torch.from_numpy(W0) - eta * W.grad).numpy()
        _, W_fin = fwd(x, ids, E, Wu, Wg, W0, T, eta)
        _close(W_fin[0], W_ref, what=f"P2 autograd step d={d} f={f} T={T}")


def block_causal_closed_form(x, ids_row, E, Wu, Wg, W0, C, eta):
    """y = Z W0^T + eta (M * Z Z^T) V with M[t,s] = 1 iff s//C < t//C;
    W_final = W0 + eta V^T Z (block-causal linear attention form)."""
    Z = _torch_z(x, Wu, Wg).numpy()
    V = _torch_v(ids_row, E).numpy()
    T = Z.shape[0]
    t = np.arange(T)
    M = (t[None, :] // C) < (t[:, None] // C)
    y = Z @ W0.T + eta * ((M * (Z @ Z.T)) @ V)
    return y, W0 + eta * V.T @ Z


# P3: multi-chunk closed form, several C including ragged last chunks.
def check_closed_form(fwd, seed=2):
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=6, f=10, B=2, T=23)
    eta = 0.21
    for C in (1, 2, 3, 5, 8, 23, 40):
        y, W = fwd(x, ids, E, Wu, Wg, W0, C, eta)
        for b in range(2):
            y_ref, W_ref = block_causal_closed_form(x[b], ids[b], E, Wu, Wg, W0, C, eta)
            _close(y[b], y_ref, 1e-9, what=f"P3 C={C} b={b} y")
            _close(W[b], W_ref, 1e-9, what=f"P3 C={C} b={b} W_final")


# P4: explicit parallel prefix form (all deltas, exclusive cumulative sum, then
# outputs) and, for C = 1, the per-token rule.
def check_prefix_and_per_token(fwd, seed=3):
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=5, f=9, B=1, T=17)
    eta = 0.3
    Z = _torch_z(x[0], Wu, Wg).numpy()
    V = _torch_v(ids[0], E).numpy()
    for C in (3, 4, 7):
        starts = list(range(0, 17, C))
        deltas = [eta * V[s:s + C].T @ Z[s:s + C] for s in starts]
        prefix = np.cumsum(np.stack([np.zeros_like(W0)] + deltas), axis=0)  # exclusive
        y_ref = np.concatenate([Z[s:s + C] @ (W0 + prefix[i]).T for i, s in enumerate(starts)])
        y, W = fwd(x, ids, E, Wu, Wg, W0, C, eta)
        _close(y[0], y_ref, 1e-9, what=f"P4 prefix C={C} y")
        _close(W[0], W0 + prefix[-1], 1e-9, what=f"P4 prefix C={C} W_final")
    Wt = W0.copy()
    y_tok = np.zeros((17, 5))
    for t in range(17):
        y_tok[t] = Wt @ Z[t]
        Wt = Wt + eta * np.outer(V[t], Z[t])
    y, W = fwd(x, ids, E, Wu, Wg, W0, 1, eta)
    _close(y[0], y_tok, 1e-9, what="P4 per-token y")
    _close(W[0], Wt, 1e-9, what="P4 per-token W_final")


# P5: causality. Chunk i's output ignores x after chunk i and ids after position iC;
# the one-token shift makes chunk i+1 depend on ids[(i+1)C].
def check_causality(fwd, seed=4):
    rng = np.random.default_rng(seed)
    C, T = 4, 16
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=6, f=10, B=1, T=T)
    eta = 0.5
    y0, _ = fwd(x, ids, E, Wu, Wg, W0, C, eta)
    for i in range(T // C):
        end = (i + 1) * C
        x2 = x.copy()
        x2[0, end:] += rng.standard_normal(x2[0, end:].shape)
        ids2 = ids.copy()
        ids2[0, i * C + 1:] = (ids2[0, i * C + 1:] + 1 + rng.integers(0, 7, T - i * C)) % E.shape[0]
        y1, _ = fwd(x2, ids, E, Wu, Wg, W0, C, eta)
        y2, _ = fwd(x, ids2, E, Wu, Wg, W0, C, eta)
        assert np.array_equal(y1[0, :end], y0[0, :end]), f"P5 x after chunk {i} leaked"
        assert np.array_equal(y2[0, :end], y0[0, :end]), f"P5 ids after {i * C} leaked into chunk {i}"
    for i in range(T // C - 1):
        ids3 = ids.copy()
        ids3[0, (i + 1) * C] = (ids3[0, (i + 1) * C] + 3) % E.shape[0]
        y3, _ = fwd(x, ids3, E, Wu, Wg, W0, C, eta)
        s = (i + 1) * C
        assert np.array_equal(y3[0, :s], y0[0, :s]), "P5 shifted id leaked backwards"
        assert not np.allclose(y3[0, s:s + C], y0[0, s:s + C], rtol=0, atol=1e-12), \
            f"P5 chunk {i + 1} must see the target built from ids[{s}]"


# P6: linearity in eta of y - y(0) and W_final - W0.
def check_linearity(fwd, seed=5):
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=6, f=10, B=1, T=15)
    y0, _ = fwd(x, ids, E, Wu, Wg, W0, 4, 0.0)
    y1, W1 = fwd(x, ids, E, Wu, Wg, W0, 4, 0.1)
    y3, W3 = fwd(x, ids, E, Wu, Wg, W0, 4, 0.3)
    _close(y3 - y0, 3.0 * (y1 - y0), 1e-9, what="P6 y linear in eta")
    _close(W3 - W0, 3.0 * (W1 - W0), 1e-9, what="P6 W linear in eta")


# P7: two calls (T1 a multiple of C, look-ahead id passed) equal one call.
def check_segments(fwd, seed=6):
    rng = np.random.default_rng(seed)
    C, T = 3, 14
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=6, f=10, B=2, T=T)
    y, W = fwd(x, ids, E, Wu, Wg, W0, C, 0.4)
    for T1 in (3, 6, 12):
        ya, Wa = fwd(x[:, :T1], ids[:, :T1 + 1], E, Wu, Wg, W0, C, 0.4)
        yb, Wb = fwd(x[:, T1:], ids[:, T1:], E, Wu, Wg, Wa, C, 0.4)
        _close(np.concatenate([ya, yb], axis=1), y, 1e-12, what=f"P7 split at {T1} y")
        _close(Wb, W, 1e-12, what=f"P7 split at {T1} W_final")


# P9: sequences are independent; each keeps its own state.
def check_batch_independence(fwd, seed=7):
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=6, f=10, B=3, T=11)
    Wb = np.stack([W0, 0.5 * W0, -W0])
    y, W = fwd(x, ids, E, Wu, Wg, Wb, 4, 0.2)
    for b in range(3):
        y1, W1 = fwd(x[b:b + 1], ids[b:b + 1], E, Wu, Wg, Wb[b], 4, 0.2)
        assert np.array_equal(y1[0], y[b]) and np.array_equal(W1[0], W[b]), f"P9 sequence {b}"


# P10: induction direction. Tokens A B in chunk 0 and A again in chunk 1: the
# LM-aligned update raises B's logit for the repeated A (the pages' Theorem 1
# setting); the change equals eta * sum_t <e_B, v_t> <z_t, z_A>.
def check_induction(fwd, seed=8):
    rng = np.random.default_rng(seed)
    d, f, vocab, C = 64, 96, 40, 8
    emb = rng.standard_normal((vocab, d))           # token -> layer input
    E = rng.standard_normal((vocab, d)) / np.sqrt(d)  # near-orthogonal target rows
    Wu = rng.standard_normal((f, d)) / np.sqrt(d)
    Wg = rng.standard_normal((f, d)) / np.sqrt(d)
    W0 = rng.standard_normal((d, f)) / np.sqrt(f)
    A, Btok = 3, 17
    toks = rng.integers(20, vocab, size=2 * C + 1)
    toks[2], toks[3] = A, Btok          # "A B" inside chunk 0
    toks[C + 4] = A                     # A again in chunk 1
    x = emb[toks[:-1]][None]
    ids = toks[None].astype(np.int32)
    eta = 0.05
    y, _ = fwd(x, ids, E, Wu, Wg, W0, C, eta)
    y_static, _ = fwd(x, ids, E, Wu, Wg, W0, C, 0.0)
    delta = y[0, C + 4] - y_static[0, C + 4]
    Z = _torch_z(x[0], Wu, Wg).numpy()
    V = _torch_v(ids[0], E).numpy()
    expect = eta * sum(np.dot(E[Btok], V[t]) * np.dot(Z[t], Z[C + 4]) for t in range(C))
    got = float(E[Btok] @ delta)
    assert abs(got - expect) <= 1e-9 * max(1.0, abs(expect)), f"P10 logit change {got} vs {expect}"
    assert got > 0, "P10 the repeated key must raise the logit of the token that followed it"
    others = [float(E[w] @ delta) for w in range(vocab) if w not in (Btok,)]
    assert got > np.max(np.abs(others)), "P10 B's logit change must dominate the others"


# Zero-target padding: ids outside [0, vocab) give zero target rows.
def check_zero_targets(fwd, seed=9):
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=6, f=10, B=1, T=9)
    bad = np.full_like(ids, -1)
    bad[0, 0] = 2
    bad[0, 5] = E.shape[0]
    y, W = fwd(x, bad, E, Wu, Wg, W0, 3, 0.7)
    y_ref = (_torch_z(x, Wu, Wg) @ torch.from_numpy(W0).T).numpy()
    _close(y, y_ref, what="zero targets y")
    _close(W[0], W0, what="zero targets W_final")
    # only the look-ahead id is invalid: the last row's target is zero
    ids2 = ids.copy()
    ids2[0, -1] = -5
    _, W2 = fwd(x, ids2, E, Wu, Wg, W0, 3, 0.7)
    Z = _torch_z(x[0], Wu, Wg).numpy()
    V = _torch_v(np.concatenate([ids[0, :-1], [0]]), E).numpy()
    V[-1] = 0.0
    _close(W2[0], W0 + 0.7 * V.T @ Z, 1e-9, what="zero look-ahead W_final")


# P11: update clipping (paperlayer App. C.2 "Inference Stability"; iplexlaw
# sec. 6). The reference takes each chunk's norm through the chunk Grams,
# ||V_i^T Z_i||_F^2 = sum((V_i V_i^T) * (Z_i Z_i^T)), not through the update
# matrix itself, and applies the factors in the block-causal closed form.
def clipped_closed_form(x, ids_row, E, Wu, Wg, W0, C, eta, tau):
    Z = _torch_z(x, Wu, Wg).numpy()
    V = _torch_v(ids_row, E).numpy()
    T = Z.shape[0]
    cidx = np.arange(T) // C
    n_chunks = int(cidx.max()) + 1
    c = np.ones(n_chunks)
    norms = np.zeros(n_chunks)
    for i in range(n_chunks):
        sel = cidx == i
        Zi, Vi = Z[sel], V[sel]
        norms[i] = eta * np.sqrt(max(float(np.sum((Vi @ Vi.T) * (Zi @ Zi.T))), 0.0))
        if norms[i] > tau:
            c[i] = tau / norms[i]
    M = (cidx[None, :] < cidx[:, None]) * c[cidx][None, :]
    y = Z @ W0.T + eta * ((M * (Z @ Z.T)) @ V)
    W = W0 + eta * (V * c[cidx][:, None]).T @ Z
    return y, W, c, norms


def check_clip_closed_form(fwd, seed=12):
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=6, f=10, B=2, T=23)
    eta = 0.21
    clipped = kept = 0
    for C in (1, 3, 5, 23):
        norms = np.concatenate([clipped_closed_form(x[b], ids[b], E, Wu, Wg, W0, C, eta, np.inf)[3]
                                for b in range(2)])
        tau = float(np.median(norms)) if len(norms) > 2 else 0.5 * float(norms.min())
        y, W = fwd(x, ids, E, Wu, Wg, W0, C, eta, clip_tau=tau)
        for b in range(2):
            y_ref, W_ref, c, _ = clipped_closed_form(x[b], ids[b], E, Wu, Wg, W0, C, eta, tau)
            clipped += int(np.sum(c < 1))
            kept += int(np.sum(c == 1))
            _close(y[b], y_ref, 1e-9, what=f"P11 C={C} b={b} y")
            _close(W[b], W_ref, 1e-9, what=f"P11 C={C} b={b} W_final")
    assert clipped > 0 and kept > 0


def check_clip_limits(fwd, seed=13):
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=5, f=8, B=1, T=16)
    eta = 0.4
    # an infinite threshold never clips
    y0, W0_ = fwd(x, ids, E, Wu, Wg, W0, 4, eta)
    y1, W1 = fwd(x, ids, E, Wu, Wg, W0, 4, eta, clip_tau=np.inf)
    assert np.array_equal(y0, y1) and np.array_equal(W0_, W1), "P11 tau=inf changed the result"
    # a vanishing threshold leaves the textbook static MLP
    y2, W2 = fwd(x, ids, E, Wu, Wg, W0, 4, eta, clip_tau=1e-300)
    Z = _torch_z(x[0], Wu, Wg).numpy()
    _close(y2[0], Z @ W0.T, 1e-12, what="P11 tau->0 y")
    assert np.max(np.abs(W2[0] - W0)) <= 1e-290
    # chunk by chunk: each applied update is the raw update scaled to norm min(norm, tau)
    tau = 0.8 * float(np.min(clipped_closed_form(x[0], ids[0], E, Wu, Wg, W0, 4, eta, np.inf)[3]))
    tau = max(tau, 1e-3)
    W = W0.copy()
    n_clipped = 0
    for s in range(0, 16, 4):
        xs, ids_s = x[:, s:s + 4], ids[:, s:s + 5]
        _, Wn = fwd(xs, ids_s, E, Wu, Wg, W, 4, eta, clip_tau=tau)
        _, Wr = fwd(xs, ids_s, E, Wu, Wg, W, 4, eta)
        d_app, d_raw = Wn[0] - W, Wr[0] - W
        n_raw = np.linalg.norm(d_raw)
        _close(d_app, d_raw * (min(1.0, tau / n_raw) if n_raw > 0 else 1.0), 1e-9,
               what=f"P11 chunk at {s} applied update")
        assert abs(np.linalg.norm(d_app) - min(n_raw, tau)) <= 1e-9 * max(n_raw, tau)
        n_clipped += int(n_raw > tau)
        W = Wn[0]
    assert n_clipped > 0


# P12: the general target V^ = Conv1D(X0) W_target (paperlayer sec. 3
# "LM-Aligned Objective"; iplexlaw sec. 4 and sec. 6). The reference builds it
# as banded shift matrices acting on the embedded token rows, not with a loop.
def conv_target_matrix_form(ids_row, E, conv_w, W_target, C):
    ids_row = np.asarray(ids_row)
    T = ids_row.shape[0] - 1
    X = _torch_v(np.concatenate([[-1], ids_row[1:]]), E).numpy()  # X[p-1] = embedding of ids[p]
    X = np.concatenate([np.zeros((1, E.shape[1])), X])              # X[p] = embedding of ids[p], X[0] unused
    t = np.arange(T)
    limit = np.minimum((t // C + 1) * C, T)
    U = np.zeros((T, E.shape[1]))
    for k in range(conv_w.shape[0]):
        Sk = np.zeros((T, T + 1))
        ok = t + 1 + k <= limit
        Sk[t[ok], (t + 1 + k)[ok]] = 1.0
        U += (Sk @ X) * conv_w[k][None, :]
    return U @ W_target


def _conv_case(rng, d=6, f=10, B=1, T=23, K=5):
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=d, f=f, B=B, T=T)
    cw = rng.standard_normal((K, d))
    Wt = rng.standard_normal((d, d)) / np.sqrt(d)
    return x, ids, E, Wu, Wg, W0, cw, Wt


def check_conv_target(fwd, seed=14):
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0, cw, Wt = _conv_case(rng, B=2)
    eta = 0.17
    # one tap of weight 1 and W_target = I: the next-token target
    y1, W1 = fwd(x, ids, E, Wu, Wg, W0, 5, eta, conv_w=np.ones((1, 6)), W_target=np.eye(6))
    y0, W0_ = fwd(x, ids, E, Wu, Wg, W0, 5, eta)
    _close(y1, y0, 1e-13, what="P12 one tap = next-token y")
    _close(W1, W0_, 1e-13, what="P12 one tap = next-token W_final")
    # one tap with per-channel weights folds into the table: E' = E diag(w) W_target
    w1 = cw[:1]
    y2, W2 = fwd(x, ids, E, Wu, Wg, W0, 5, eta, conv_w=w1, W_target=Wt)
    y3, W3 = fwd(x, ids, (E * w1) @ Wt, Wu, Wg, W0, 5, eta)
    _close(y2, y3, 1e-11, what="P12 folded table y")
    _close(W2, W3, 1e-11, what="P12 folded table W_final")
    # five taps, several chunk sizes: block-causal closed form on the banded-matrix target
    for C in (1, 2, 3, 5, 8, 23):
        y, W = fwd(x, ids, E, Wu, Wg, W0, C, eta, conv_w=cw, W_target=Wt)
        for b in range(2):
            Z = _torch_z(x[b], Wu, Wg).numpy()
            V = conv_target_matrix_form(ids[b], E, cw, Wt, C)
            T = Z.shape[0]
            tt = np.arange(T)
            M = (tt[None, :] // C) < (tt[:, None] // C)
            _close(y[b], Z @ W0.T + eta * ((M * (Z @ Z.T)) @ V), 1e-9, what=f"P12 C={C} b={b} y")
            _close(W[b], W0 + eta * V.T @ Z, 1e-9, what=f"P12 C={C} b={b} W_final")


def check_conv_causality(fwd, seed=15):
    # brute force: changing the token at position q leaves every output before q unchanged
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0, cw, Wt = _conv_case(rng, T=16)
    C, eta = 4, 0.3
    y, _ = fwd(x, ids, E, Wu, Wg, W0, C, eta, conv_w=cw, W_target=Wt)
    for q in range(1, 17):
        ids2 = ids.copy()
        ids2[0, q] = (ids2[0, q] + 1) % E.shape[0]
        y2, _ = fwd(x, ids2, E, Wu, Wg, W0, C, eta, conv_w=cw, W_target=Wt)
        assert np.array_equal(y2[0, :q], y[0, :q]), f"P12 causality: token {q} reached an earlier output"
        if q % C == 0 and q < 16:
            # the first token of a chunk is tapped by the previous chunk's targets
            assert not np.array_equal(y2[0, q:], y[0, q:])


# P13: packed documents (paperlayer App. B; iplexlaw sec. 6). Checked through
# the plain forward (no boundaries), the block-causal closed form on one
# document from the initial weight, and brute-force independence.
def check_documents(fwd, seed=16):
    import oracle.ttt_oracle as _ot

    def fdocs(*a, **k):
        return _ot.ttt_forward_docs(*a, **k)
    rng = np.random.default_rng(seed)
    x, ids, E, Wu, Wg, W0 = tiny_case(rng, d=5, f=8, B=2, T=22)
    Wentry = W0 + 0.1 * rng.standard_normal(W0.shape)  # a carried state, not the reset value
    C, eta = 4, 0.3
    # no boundaries: the plain forward
    y, W = fdocs(x, ids, E, Wu, Wg, Wentry, W0, C, eta, [[], []])
    y_ref, W_ref = fwd(x, ids, E, Wu, Wg, Wentry, C, eta)
    _close(y, y_ref, 1e-12, what="P13 no boundary y")
    _close(W, W_ref, 1e-12, what="P13 no boundary W_final")
    # a boundary at 9 (not a multiple of C): the last document alone from W0,
    # chunked from its own first token (closed form), its look-ahead kept
    y, W = fdocs(x, ids, E, Wu, Wg, Wentry, W0, C, eta, [[9], [6, 15]])
    for b, r in ((0, 9), (1, 15)):
        y_cf, W_cf = block_causal_closed_form(x[b, r:], ids[b, r:], E, Wu, Wg, W0, C, eta)
        _close(y[b, r:], y_cf, 1e-9, what=f"P13 last document b={b} y")
        _close(W[b], W_cf, 1e-9, what=f"P13 last document b={b} W_final")
    # the first document: from the carried state, its last target zero
    ids_z = ids.copy()
    ids_z[0, 9] = -1
    y_cf, _ = block_causal_closed_form(x[0, :9], ids_z[0, :10], E, Wu, Wg, Wentry, C, eta)
    _close(y[0, :9], y_cf, 1e-9, what="P13 first document y")
    # brute force: nothing before a boundary reaches the outputs after it
    for q in range(0, 9):
        x2 = x.copy()
        x2[0, q] += 1.0
        y2, W2 = fdocs(x2, ids, E, Wu, Wg, Wentry, W0, C, eta, [[9], [6, 15]])
        assert np.array_equal(y2[0, 9:], y[0, 9:]) and np.array_equal(W2[0], W[0])
    # the first token of the next document is no target of this one's outputs (the
    # last chunk's update, the only one it could enter, is discarded by the reset)
    ids2 = ids.copy()
    ids2[0, 9] = (ids2[0, 9] + 1) % E.shape[0]
    y2, W2 = fdocs(x, ids2, E, Wu, Wg, Wentry, W0, C, eta, [[9], [6, 15]])
    assert np.array_equal(y2[0, :9], y[0, :9]), "P13 look-ahead crossed a document end"


ALL_PINS = [
    check_static_mlp,
    lambda fwd: check_static_mlp(fwd, square=True),
    check_autograd_step,
    check_closed_form,
    check_prefix_and_per_token,
    check_causality,
    check_linearity,
    check_segments,
    check_batch_independence,
    check_induction,
    check_zero_targets,
    check_clip_closed_form,
    check_clip_limits,
    check_conv_target,
    check_conv_causality,
    check_documents,
]
