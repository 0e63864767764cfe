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
