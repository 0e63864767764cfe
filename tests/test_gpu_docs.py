"""GPU parity for packed documents with in-call resets (paperlayer App. B;
iplexlaw sec. 6): at every document start the fast weight returns to W_down0
and chunking restarts from that token. Against oracle.ttt_forward_docs;
tolerances as in the other parity tests.
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as ttt
import oracle
from synth import make_inputs, make_target_conv
from tests.gpu_util import Layer, dev, max_rel, rel_fro

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 3e-2


def _gpu(lay, starts):
    y, Wf = ttt.ttt_forward_docs(lay.h, lay.x, lay.ids, lay.E, starts, want_W_final=True)
    torch.cuda.synchronize()
    return y.double().cpu().numpy(), Wf.double().cpu().numpy()


def _ref(w, C, starts, W_entry=None, **kw):
    W0 = w.W_down0
    return oracle.ttt_forward_docs(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, W0 if W_entry is None else W_entry, W0, C,
                                   w.eta, starts, **kw)


CASES = [  # (dtype, T, C, starts)
    ("f32", 2000, 128, [[700, 1300], [1000]]),
    ("f32", 900, 1, [[1, 450, 899], []]),
    ("f32", 1500, 100, [[512], [3, 1000, 1001]]),
    ("bf16", 3000, 128, [[700, 1300], [1000]]),
    ("bf16", 2500, 256, [[1, 2499], [1024, 2048]]),
    ("bf16", 2000, 24, [[1000], [37, 999, 1500]]),
]


@pytest.mark.parametrize("dtype,T,C,starts", CASES)
def test_docs(dtype, T, C, starts):
    d, f, eta = (64, 192, 0.02) if dtype == "f32" else (256, 512, 1e-3)
    w = make_inputs(d=d, f=f, B=2, T=T, C=C, eta=eta, dtype=dtype, vocab=151, e_std=1.0, seed=100 + T + C)
    print(f"[docs {dtype}] T={T} C={C} starts={starts}", flush=True)
    y, Wf = _gpu(Layer(w), starts)
    y_ref, W_ref = _ref(w, C, starts)
    metric, tol = (max_rel, F32_TOL) if dtype == "f32" else (rel_fro, BF16_TOL)
    assert metric(y, y_ref) <= tol, metric(y, y_ref)
    assert metric(Wf, W_ref) <= tol, metric(Wf, W_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_docs_continue_carried_state_with_clip_and_target(dtype):
    # a plain call first; the packed call's first document continues that state
    d, f, eta = (64, 192, 0.02) if dtype == "f32" else (256, 512, 1e-3)
    w = make_inputs(d=d, f=f, B=2, T=2400, C=100, eta=eta, dtype=dtype, vocab=151, e_std=1.0, seed=120)
    cw, Wt = make_target_conv(d, 5, dtype, seed=12)
    lay = Layer(w)
    ttt.ttt_set_target_conv(lay.h, dev(cw, lay.dt), dev(Wt, lay.dt))
    T1 = 1000
    x1, ids1 = lay.x[:, :T1].contiguous(), lay.ids[:, :T1 + 1].contiguous()
    ttt.ttt_forward_chunked(lay.h, x1, ids1, lay.E)
    _, W_mid = oracle.ttt_forward(w.x[:, :T1], w.ids[:, :T1 + 1], w.E_tgt, w.W_up, w.W_gate, w.W_down0, 100, eta,
                                  conv_w=cw, W_target=Wt)
    rest = [[300, 900], [150]]
    tau = 0.3 * float(np.median([np.linalg.norm(W_mid[b] - w.W_down0) for b in range(2)])) / np.sqrt(10)
    ttt.ttt_set_clip(lay.h, tau)
    x2, ids2 = lay.x[:, T1:].contiguous(), lay.ids[:, T1:].contiguous()
    y, Wf = ttt.ttt_forward_docs(lay.h, x2, ids2, lay.E, rest, want_W_final=True)
    torch.cuda.synchronize()
    y_ref, W_ref = oracle.ttt_forward_docs(w.x[:, T1:], w.ids[:, T1:], w.E_tgt, w.W_up, w.W_gate, W_mid, w.W_down0,
                                           100, eta, rest, clip_tau=tau, conv_w=cw, W_target=Wt)
    metric, tol = (max_rel, F32_TOL) if dtype == "f32" else (rel_fro, BF16_TOL)
    y, Wf = y.double().cpu().numpy(), Wf.double().cpu().numpy()
    assert metric(y, y_ref) <= tol, metric(y, y_ref)
    assert metric(Wf, W_ref) <= tol, metric(Wf, W_ref)


def test_docs_without_boundaries_is_plain_forward_and_errors():
    w = make_inputs(d=256, f=256, B=2, T=700, C=64, eta=2e-3, dtype="bf16", vocab=77, e_std=1.0, seed=130)
    lay = Layer(w)
    y0, W0 = lay.forward()
    y0, W0 = y0.clone(), W0.clone()
    ttt.ttt_reset(lay.h)
    y1, W1 = ttt.ttt_forward_docs(lay.h, lay.x, lay.ids, lay.E, [[], []], want_W_final=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(W1, W0)
    for bad in ([[300, 200], []], [[0], []], [[700], []]):
        with pytest.raises(ttt.TTTError) as e:
            ttt.ttt_forward_docs(lay.h, lay.x, lay.ids, lay.E, bad)
        assert e.value.code == -7


def test_docs_many_documents_one_launch_sequence():
    """64 documents of 2048 tokens across two sequences, at the 1k/4k layer width. On a bf16 handle (plain
    target, no clipping) a packed call runs every document as a sequence of its own in one launch sequence;
    each document then gives the same bits as a call of its own from a reset state, and matches the oracle."""
    T, C, ndoc = 32 * 2048, 256, 32
    w = make_inputs(d=1024, f=4096, B=2, T=T, C=C, eta=1e-3, dtype="bf16", vocab=4096, e_std=0.02, seed=140)
    starts = [[2048 * k for k in range(1, ndoc)] for _ in range(2)]
    print(f"[docs many] B=2 T={T} C={C}, {ndoc} documents of 2048 per sequence", flush=True)
    lay = Layer(w)
    ttt.ttt_set_profiling(lay.h, True)
    y, Wf = ttt.ttt_forward_docs(lay.h, lay.x, lay.ids, lay.E, starts, want_W_final=True)
    torch.cuda.synchronize()
    ph = ttt.ttt_phase_times(lay.h)
    assert all(v >= 0.0 for v in ph)
    # documents 0, 1 and the last of sequence 1, each alone from a reset state (its look-ahead id kept)
    for j in (0, 1, ndoc - 1):
        s0 = 2048 * j
        ttt.ttt_reset(lay.h)
        xs = lay.x[1:2, s0:s0 + 2048].contiguous()
        ids_s = lay.ids[1:2, s0:s0 + 2049].contiguous()
        ys, Ws = ttt.ttt_forward_chunked(lay.h, xs, ids_s, lay.E, want_W_final=True)
        torch.cuda.synchronize()
        assert torch.equal(ys[0], y[1, s0:s0 + 2048]), f"document {j}"
        if j == ndoc - 1:
            assert torch.equal(Ws[0], Wf[1])
    y_ref, W_ref = _ref(w, C, starts)
    y, Wf = y.double().cpu().numpy(), Wf.double().cpu().numpy()
    W0 = w.W_down0.astype(np.float64)
    e = (rel_fro(y, y_ref), rel_fro(Wf, W_ref), rel_fro(Wf - W0, W_ref - W0))
    print(f"  y err {e[0]:.2e}, W_final err {e[1]:.2e}, W_final - W0 err {e[2]:.2e}", flush=True)
    assert max(e) <= BF16_TOL, e


@pytest.mark.parametrize("y_f32", [False, True])
def test_docs_ragged_lengths_after_a_plain_call(y_f32):
    """Documents of 1, 255, 256, 257 ... tokens (each padded to whole 256-slot tiles inside the library), a
    sequence with no document start, and a carried state from a plain call before the packed one."""
    d, f, C, T1, T = 256, 512, 128, 700, 3000
    w = make_inputs(d=d, f=f, B=3, T=T1 + T, C=C, eta=1e-3, dtype="bf16", vocab=151, e_std=1.0, seed=150)
    lay = Layer(w)
    ttt.ttt_set_output_f32(lay.h, y_f32)
    x1, ids1 = lay.x[:, :T1].contiguous(), lay.ids[:, :T1 + 1].contiguous()
    ttt.ttt_forward_chunked(lay.h, x1, ids1, lay.E)
    _, W_mid = oracle.ttt_forward(w.x[:, :T1], w.ids[:, :T1 + 1], w.E_tgt, w.W_up, w.W_gate, w.W_down0, C, w.eta)
    starts = [[1, 2, 257, 513, 770, 1000, 2999], [256], []]
    print(f"[docs ragged] y_f32={y_f32} starts={starts}", flush=True)
    x2, ids2 = lay.x[:, T1:].contiguous(), lay.ids[:, T1:].contiguous()
    y, Wf = ttt.ttt_forward_docs(lay.h, x2, ids2, lay.E, starts, want_W_final=True)
    torch.cuda.synchronize()
    assert y.dtype == (torch.float32 if y_f32 else torch.bfloat16)
    y_ref, W_ref = oracle.ttt_forward_docs(w.x[:, T1:], w.ids[:, T1:], w.E_tgt, w.W_up, w.W_gate, W_mid, w.W_down0,
                                           C, w.eta, starts)
    y, Wf = y.double().cpu().numpy(), Wf.double().cpu().numpy()
    W0 = w.W_down0.astype(np.float64)
    e = (rel_fro(y, y_ref), rel_fro(Wf, W_ref), rel_fro(Wf[2] - W_mid[2], W_ref[2] - W_mid[2]))
    print(f"  y err {e[0]:.2e}, W_final err {e[1]:.2e}, carried sequence's update err {e[2]:.2e}", flush=True)
    assert max(e) <= BF16_TOL, e
    # the state left for the next call: sequence 2 continued its carried state; 0 and 1 end in a fresh document
    D = ttt.ttt_state_delta(lay.h, 3).double().cpu().numpy()
    assert rel_fro(D + W0, W_ref) <= BF16_TOL


@pytest.mark.parametrize("C", [100, 256])
def test_docs_many_with_clip_and_target_one_launch_sequence(C):
    """Ragged documents (1 to 700 tokens) across three sequences, with clipping and the general target
    (K = 5) on a bf16 handle: a packed call is one launch sequence here too, its chunk Grams, factors and
    target rows taken per document. C = 100 makes a chunk span two 256-slot tiles."""
    d, f, T = 256, 512, 1800
    w = make_inputs(d=d, f=f, B=3, T=T, C=C, eta=1e-3, dtype="bf16", vocab=211, e_std=1.0, seed=160 + C)
    cw, Wt = make_target_conv(d, 5, "bf16", seed=16)
    lay = Layer(w)
    ttt.ttt_set_target_conv(lay.h, dev(cw, lay.dt), dev(Wt, lay.dt))
    starts = [[1, 2, 100, 356, 700, 1400], [256, 512, 768, 1024, 1280, 1536], [700]]
    # a threshold that clips some chunk updates and not others: from the oracle's first documents
    _, W_probe = oracle.ttt_forward_docs(w.x[:, :700], w.ids[:, :701], w.E_tgt, w.W_up, w.W_gate, w.W_down0,
                                         w.W_down0, C, w.eta, [[1, 2, 100, 356], [256, 512], []], conv_w=cw,
                                         W_target=Wt)
    tau = 0.05 * float(np.median([np.linalg.norm(W_probe[b] - w.W_down0) for b in range(3)]))
    ttt.ttt_set_clip(lay.h, tau)
    print(f"[docs clip+target] C={C} tau={tau:.3e} starts={starts}", flush=True)
    y, Wf = ttt.ttt_forward_docs(lay.h, lay.x, lay.ids, lay.E, starts, want_W_final=True)
    torch.cuda.synchronize()
    y_ref, W_ref = _ref(w, C, starts, clip_tau=tau, conv_w=cw, W_target=Wt)
    y, Wf = y.double().cpu().numpy(), Wf.double().cpu().numpy()
    W0 = w.W_down0.astype(np.float64)
    e = (rel_fro(y, y_ref), rel_fro(Wf, W_ref), rel_fro(Wf - W0, W_ref - W0))
    print(f"  y err {e[0]:.2e}, W_final err {e[1]:.2e}, W_final - W0 err {e[2]:.2e}", flush=True)
    assert max(e) <= BF16_TOL, e
    # one document alone from a reset state gives the same bits (document 3 of sequence 1: positions 768 .. 1023)
    ttt.ttt_reset(lay.h)
    ys, _ = ttt.ttt_forward_chunked(lay.h, lay.x[1:2, 768:1024].contiguous(), lay.ids[1:2, 768:1025].contiguous(),
                                    lay.E)
    torch.cuda.synchronize()
    y_dev, _ = ttt.ttt_forward_docs(lay.h, lay.x, lay.ids, lay.E, starts)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], y_dev[1, 768:1024])
