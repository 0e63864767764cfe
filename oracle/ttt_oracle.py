"""CPU oracle for the chunk-wise fast-weight update of In-Place Test-Time Training.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or call this module. The product path (the HIP
library and its Python binding) never does, and shares no code with it.

What it computes is the plain definition, run sequentially in fp64 with NumPy.
For each sequence b, starting from its entry state S (the initial W_down, or
the state a previous call left):

  1. Z = SiLU(x W_gate^T) * (x W_up^T): the gated MLP's intermediate activation,
     two projections followed by a gate, with W_up and W_gate frozen
     (paperlayer.ai summary, sec. 3 "In-Place Adaptation"; iplexlaw.co.kr
     walkthrough, sec. 2; SwiGLU per the paperlayer summary, App. C.3).
  2. V[t] = E_tgt[ids[t+1]]: the LM-aligned target V^ = Conv1D(X0) W_target
     with the convolution kernel reduced to a single tap on the next token and
     W_target folded into the target-embedding table E_tgt (paperlayer sec. 3
     "LM-Aligned Objective"; iplexlaw sec. 4, where the kernel may pick "the
     next token"). A row whose id lies outside [0, vocab) is zero (the causal
     zero padding of paperlayer App. B).
  3. For chunks i = 0 .. n-1 of C consecutive tokens (the last may be short):
     y[chunk i] = Z[chunk i] S^T with the pre-update state (apply), then
     S <- S + eta * V[chunk i]^T Z[chunk i] (update) (iplexlaw sec. 3,
     apply-then-update; update rule dW_down = eta V^T Z, iplexlaw sec. 2 and
     sec. 4; paperlayer sec. 3 "Chunk-Wise Updates").
  4. Return y and the final S (inclusive of the last chunk's update).

Optional general target (conv_w, W_target): V^ = Conv1D(X0) W_target with
a depthwise kernel of K taps over the token embeddings X0 (rows of the table
passed as E_tgt), on the tokens after position t (paperlayer sec. 3
"LM-Aligned Objective"; iplexlaw sec. 4 and sec. 6, kernel size 5, "nearby
future tokens"). The chunk boundary pads the convolution: row t of chunk i
uses the embedding at position t+1+k only up to position (i+1)C (and T), the
first token of the next chunk, which that chunk already holds as its input;
anything further would let chunk i+1's first outputs see later tokens
(iplexlaw sec. 6, padding at chunk boundaries; paperlayer App. B, causal
padding). With K = 1, conv_w = 1 and W_target = I it is the next-token target
of step 2.

Optional update clipping (clip_tau): before a chunk's update is applied it is
rescaled to Frobenius norm tau when its norm exceeds tau, i.e.
dW <- dW * min(1, tau / ||dW||_F), with dW = eta V[chunk]^T Z[chunk] the
whole chunk update (paperlayer App. C.2 "Inference Stability", where the
threshold for the reported long-context evaluations is 1e-5; iplexlaw sec. 6,
the closing implementation notes). Off by default.

Readings of points the pages leave open (kept identical on both sides):
  - the update is the sum over the chunk's tokens (no 1/C), sign "+";
  - the one-token shift crosses chunk boundaries (the last row of chunk i takes
    token (i+1)C, which every later chunk already sees as input);
  - no biases, no normalisation of Z or V;
  - clipping, when on, acts on each chunk's update as a whole (the "delta" of
    the pages), after the learning rate is applied.

Every function here is pinned by the CPU tests against closed forms, autograd,
textbook special cases and invariants; none is "parity unpinned".
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), elementwise, fp64."""
    g = _f64(g)
    return g / (1.0 + np.exp(-g))


def gated_activation(x: np.ndarray, W_up: np.ndarray, W_gate: np.ndarray) -> np.ndarray:
    """Step 1: Z = SiLU(x W_gate^T) * (x W_up^T).

    x [..., d]; W_up, W_gate [f][d] (row-major, one row per hidden unit).
    Returns Z [..., f] in fp64. The SiLU sits on the gate path.
    """
    x = _f64(x)
    u = x @ _f64(W_up).T
    g = x @ _f64(W_gate).T
    return silu(g) * u


def ntp_targets(ids: np.ndarray, E_tgt: np.ndarray) -> np.ndarray:
    """Step 2: the next-token target rows.

    ids [T+1] (position-aligned token ids plus one look-ahead id);
    E_tgt [vocab][d]. Returns V [T][d] with V[t] = E_tgt[ids[t+1]], or a zero
    row where ids[t+1] lies outside [0, vocab).
    """
    ids = np.asarray(ids)
    E = _f64(E_tgt)
    vocab, d = E.shape
    T = ids.shape[0] - 1
    V = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        tok = int(ids[t + 1])
        if 0 <= tok < vocab:
            V[t] = E[tok]
    return V


def conv_targets(ids: np.ndarray, E_in: np.ndarray, conv_w: np.ndarray, W_target: np.ndarray, C: int) -> np.ndarray:
    """The general target rows V^ = Conv1D(X0) W_target of one sequence.

    ids [T+1]; E_in [vocab][d] (token embeddings X0); conv_w [K][d] (depthwise,
    tap k on position t+1+k); W_target [d][d]. Tap k of row t is used when
    t+1+k <= min((t//C + 1) * C, T) and the id is in [0, vocab); otherwise that
    tap is zero padding. Returns V [T][d] = U W_target with U the tap sums.
    """
    ids = np.asarray(ids)
    E = _f64(E_in)
    cw = _f64(conv_w)
    vocab, d = E.shape
    T = ids.shape[0] - 1
    U = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        limit = min((t // C + 1) * C, T)  # last embedding position row t may read
        for k in range(cw.shape[0]):
            p = t + 1 + k
            if p > limit:
                break
            tok = int(ids[p])
            if 0 <= tok < vocab:
                U[t] += cw[k] * E[tok]
    return U @ _f64(W_target)


def chunk_ranges(T: int, C: int) -> List[Tuple[int, int]]:
    """Non-overlapping chunks [start, end) of C tokens covering [0, T); the last may be short."""
    if C < 1:
        raise ValueError("chunk size must be >= 1")
    return [(s, min(s + C, T)) for s in range(0, T, C)]


def clip_update(dW: np.ndarray, clip_tau: Optional[float]) -> np.ndarray:
    """Rescale one chunk update to Frobenius norm clip_tau if it is larger
    (paperlayer App. C.2; iplexlaw sec. 6). clip_tau None: unchanged."""
    if clip_tau is None:
        return dW
    n = float(np.linalg.norm(dW))  # Frobenius norm of the whole matrix
    if n > clip_tau:
        return dW * (clip_tau / n)
    return dW


def ttt_forward_one(x: np.ndarray, ids: np.ndarray, E_tgt: np.ndarray, W_up: np.ndarray,
                    W_gate: np.ndarray, W_entry: np.ndarray, C: int, eta: float,
                    clip_tau: Optional[float] = None, conv_w: Optional[np.ndarray] = None,
                    W_target: Optional[np.ndarray] = None):
    """Steps 1-4 for one sequence: x [T][d], ids [T+1], W_entry [d][f].

    clip_tau: None, or the Frobenius threshold of each chunk update.
    conv_w [K][d], W_target [d][d]: the general target (E_tgt then holds the
    token embeddings X0); None: the next-token target rows of E_tgt.
    Returns (y [T][d], W_final [d][f]) in fp64.
    """
    x = _f64(x)
    T = x.shape[0]
    S = _f64(W_entry).copy()
    y = np.zeros((T, S.shape[0]), dtype=np.float64)
    if T == 0:
        return y, S
    Z = gated_activation(x, W_up, W_gate)
    if conv_w is None:
        V = ntp_targets(ids, E_tgt)
    else:
        V = conv_targets(ids, E_tgt, conv_w, W_target, C)
    for (s, e) in chunk_ranges(T, C):
        y[s:e] = Z[s:e] @ S.T                      # apply with the pre-update state
        dW = eta * (V[s:e].T @ Z[s:e])             # the chunk's rank-C update
        S = S + clip_update(dW, clip_tau)          # then applied (clipped if asked)
    return y, S


def ttt_forward(x: np.ndarray, ids: np.ndarray, E_tgt: np.ndarray, W_up: np.ndarray,
                W_gate: np.ndarray, W_entry: np.ndarray, C: int, eta: float,
                clip_tau: Optional[float] = None, conv_w: Optional[np.ndarray] = None,
                W_target: Optional[np.ndarray] = None):
    """Batched form: x [B][T][d], ids [B][T+1], W_entry [d][f] (shared entry
    state) or [B][d][f] (one state per sequence). Each sequence is independent.

    Returns (y [B][T][d], W_final [B][d][f]) in fp64.
    """
    x = _f64(x)
    B = x.shape[0]
    W_entry = _f64(W_entry)
    ys, Ws = [], []
    for b in range(B):
        Wb = W_entry if W_entry.ndim == 2 else W_entry[b]
        yb, Sb = ttt_forward_one(x[b], ids[b], E_tgt, W_up, W_gate, Wb, C, eta, clip_tau, conv_w, W_target)
        ys.append(yb)
        Ws.append(Sb)
    return np.stack(ys), np.stack(Ws)


def ttt_forward_docs(x: np.ndarray, ids: np.ndarray, E_tgt: np.ndarray, W_up: np.ndarray, W_gate: np.ndarray,
                     W_entry: np.ndarray, W_reset: np.ndarray, C: int, eta: float,
                     doc_starts: Sequence[Sequence[int]], clip_tau: Optional[float] = None,
                     conv_w: Optional[np.ndarray] = None, W_target: Optional[np.ndarray] = None):
    """Packed documents: the stream of sequence b holds several documents, a new
    one starting at each position of doc_starts[b] (strictly increasing, inside
    (0, T)). At each document start the fast weight returns to W_reset (the
    initial W_down) and chunking restarts from that token. The last token of a
    document gets no look-ahead (its target is zero); that row lies in the
    document's last chunk, whose update the reset discards, so the choice
    never reaches an output. The call's last document keeps ids[T], the stream
    continuing into the next call
    (paperlayer App. B and iplexlaw sec. 6: reset at document boundaries so no
    state crosses between independent documents).

    x [B][T][d], ids [B][T+1], W_entry [d][f] or [B][d][f] (state at the call's
    first token). Returns (y [B][T][d], W_final [B][d][f]) in fp64.
    """
    x = _f64(x)
    B, T = x.shape[0], x.shape[1]
    W_entry = _f64(W_entry)
    ys, Ws = [], []
    for b in range(B):
        S = (W_entry if W_entry.ndim == 2 else W_entry[b]).copy()
        starts = list(doc_starts[b])
        bounds = [0] + starts + [T]
        yb = np.zeros((T, S.shape[0]))
        for j in range(len(bounds) - 1):
            s0, s1 = bounds[j], bounds[j + 1]
            if j > 0:
                S = _f64(W_reset).copy()        # a new document starts from the initial weight
            ids_seg = np.array(ids[b][s0:s1 + 1], copy=True)
            if j < len(bounds) - 2:
                ids_seg[-1] = -1                 # no look-ahead past a document's end
            yb[s0:s1], S = ttt_forward_one(x[b, s0:s1], ids_seg, E_tgt, W_up, W_gate, S, C, eta,
                                           clip_tau, conv_w, W_target)
        ys.append(yb)
        Ws.append(S)
    return np.stack(ys), np.stack(Ws)


def final_state_columns(x: np.ndarray, ids: np.ndarray, E_tgt: np.ndarray, W_up: np.ndarray,
                        W_gate: np.ndarray, W_entry: np.ndarray, C: int, eta: float,
                        cols: Sequence[int]) -> np.ndarray:
    """The final state restricted to hidden units `cols`, for one sequence.

    The update of column b of the state only involves column b of Z (the
    product V^T Z is taken column by column), so the same chunk loop as in
    ttt_forward_one, run on Z[:, cols] alone, gives W_final[:, cols] exactly.
    This makes the full-length final state checkable at sizes where the whole
    of Z is too costly to form on the host.

    x [T][d], ids [T+1], W_entry [d][f]; returns [d][len(cols)] in fp64.
    Unclipped updates only: a clipped update's scale depends on every column.
    """
    cols = list(cols)
    x = _f64(x)
    T = x.shape[0]
    Wu = _f64(W_up)[cols]
    Wg = _f64(W_gate)[cols]
    S = _f64(W_entry)[:, cols].copy()
    if T == 0:
        return S
    Zc = gated_activation(x, Wu, Wg)
    V = ntp_targets(ids, E_tgt)
    for (s, e) in chunk_ranges(T, C):
        S = S + eta * (V[s:e].T @ Zc[s:e])
    return S



def window_outputs(x: np.ndarray, ids: np.ndarray, E_tgt: np.ndarray, W_up: np.ndarray, W_gate: np.ndarray,
                   W_entry: np.ndarray, C: int, eta: float, t0: int, t1: int, block: int = 8192) -> np.ndarray:
    """The outputs y[t0:t1] of one sequence (plain next-token target, no clipping).

    The state that chunk i applies is the entry state plus the updates of
    every earlier chunk, W_entry + eta * sum_{s < iC} v_s z_s^T (the exclusive
    prefix of the chunk deltas, paperlayer App. B; iplexlaw sec. 6). With c0
    the start of the chunk holding t0, that prefix is split at c0:
      y_t = z_t (W_entry + D)^T + eta * sum_{c0 <= s < start of t's chunk} <z_t, z_s> v_s,
      D   = eta * V[:c0]^T Z[:c0],
    and D is summed over blocks of `block` tokens, so a window late in a long
    stream is reached without holding all of Z. Exact up to fp64 rounding
    order; it agrees with ttt_forward_one on y[t0:t1].

    x [T][d], ids [T+1], W_entry [d][f]; returns [t1 - t0][d] in fp64.
    """
    x = np.asarray(x)
    T = x.shape[0]
    if not (0 <= t0 <= t1 <= T):
        raise ValueError("need 0 <= t0 <= t1 <= T")
    S = _f64(W_entry)
    c0 = (t0 // C) * C
    D = np.zeros_like(S)
    for a in range(0, c0, block):
        b = min(a + block, c0)
        Zb = gated_activation(x[a:b], W_up, W_gate)
        Vb = ntp_targets(ids[a:b + 1], E_tgt)
        D += eta * (Vb.T @ Zb)
    Zw = gated_activation(x[c0:t1], W_up, W_gate)      # tokens c0 .. t1-1
    Vw = ntp_targets(ids[c0:t1 + 1], E_tgt)
    y = Zw[t0 - c0:] @ (S + D).T
    G = Zw[t0 - c0:] @ Zw.T                             # <z_t, z_s> for t in the window, s in [c0, t1)
    for r, t in enumerate(range(t0, t1)):
        n = (t // C) * C - c0                           # tokens of [c0, t1) in earlier chunks than t's
        if n > 0:
            y[r] += eta * (G[r, :n] @ Vw[:n])
    return y
