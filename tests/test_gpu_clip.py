"""GPU parity for update clipping: each chunk update rescaled to Frobenius
norm tau when larger (paperlayer App. C.2 "Inference Stability"; iplexlaw
sec. 6), against the oracle run with the same threshold.

The threshold is half the lower quartile of the unclipped chunk-update norms:
most chunks are clipped, to at most half their size (where the norms vary a
lot, as at C = 1, some are not); each case also checks that clipping changes
the result materially. Tolerances as in the other parity tests: fp32
<= 1e-4 max-relative, bf16 <= 3e-2 relative Frobenius, the latter also on the
fast-weight contributions y - y(eta=0) and W_final - W_entry.
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as ttt
import oracle
from synth import make_config, make_inputs
from tests.gpu_util import Layer, max_rel, rel_fro

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 3e-2


def _clip_threshold(w, C, T=None):
    """Half the lower quartile of the norms of the unclipped chunk updates eta V_i^T Z_i (fp64)."""
    T = w.T if T is None else T
    norms = []
    for b in range(w.B):
        Z = oracle.gated_activation(w.x[b, :T], w.W_up, w.W_gate)
        V = oracle.ntp_targets(w.ids[b, :T + 1], w.E_tgt)
        for (s, e) in oracle.chunk_ranges(T, C):
            norms.append(abs(w.eta) * np.linalg.norm(V[s:e].T @ Z[s:e]))
    return 0.5 * float(np.quantile(norms, 0.25))


def _run(w, C, G, tau, eta=None):
    lay = Layer(w, C=C, G=G, eta=eta)
    ttt.ttt_set_clip(lay.h, tau)
    return lay.forward_np()


def _check(w, C, G, tol, metric):
    tau = _clip_threshold(w, C)
    y, Wf = _run(w, C, G, tau)
    y_ref, W_ref = oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, C, w.eta, clip_tau=tau)
    _, W_raw = oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, C, w.eta)
    W0 = w.W_down0.astype(np.float64)
    print(f"  tau={tau:.3e} y err {metric(y, y_ref):.2e} W err {metric(Wf, W_ref):.2e}", flush=True)
    # clipping changes the accumulated update materially
    assert np.linalg.norm(W_ref - W_raw) > 0.01 * np.linalg.norm(W_raw - W0)
    assert metric(y, y_ref) <= tol, metric(y, y_ref)
    assert metric(Wf, W_ref) <= tol, metric(Wf, W_ref)
    return y, Wf, y_ref, W_ref, W0


FP32_CASES = [  # (T, C, G, B)
    (1000, 100, 0, 2),
    (640, 1, 0, 1),
    (1300, 8, 16, 1),
    (777, 128, 0, 1),
]


@pytest.mark.parametrize("T,C,G,B", FP32_CASES)
def test_clip_fp32(T, C, G, B):
    w = make_inputs(d=64, f=192, B=B, T=T, C=C, eta=0.02, dtype="f32", vocab=97, e_std=1.0, seed=40 + T)
    print(f"[clip fp32] T={T} C={C} G={G} B={B}", flush=True)
    _check(w, C, G, F32_TOL, max_rel)


def test_clip_fp32_single_chunk():
    # C >= T: the one chunk's update is clipped (only W_final sees it)
    w = make_inputs(d=64, f=192, B=1, T=500, C=600, eta=0.02, dtype="f32", vocab=97, e_std=1.0, seed=45)
    _, W_raw = oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, 600, w.eta)
    tau = 0.5 * float(np.linalg.norm(W_raw[0] - w.W_down0))
    y, Wf = _run(w, 600, 0, tau)
    y_ref, W_ref = oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, 600, w.eta, clip_tau=tau)
    assert max_rel(y, y_ref) <= F32_TOL
    assert max_rel(Wf, W_ref) <= F32_TOL
    assert abs(np.linalg.norm(Wf[0] - w.W_down0) - tau) <= 1e-3 * tau


BF16_CASES = [  # (T, C, G, B)
    (3000, 128, 0, 2),
    (2500, 24, 0, 1),
    (1500, 1, 0, 1),
    (4096, 512, 0, 1),
    (3000, 100, 0, 1),
    (2100, 1024, 0, 1),
]


@pytest.mark.parametrize("T,C,G,B", BF16_CASES)
def test_clip_bf16(T, C, G, B):
    w = make_inputs(d=256, f=512, B=B, T=T, C=C, eta=1e-3, dtype="bf16", vocab=301, e_std=1.0, seed=50 + T + C)
    print(f"[clip bf16] T={T} C={C} G={G} B={B}", flush=True)
    y, Wf, y_ref, W_ref, W0 = _check(w, C, G, BF16_TOL, rel_fro)
    y0, _ = Layer(w, C=C, G=G, eta=0.0).forward_np()
    y0_ref, _ = oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, C, 0.0)
    assert rel_fro(y - y0, y_ref - y0_ref) <= BF16_TOL, rel_fro(y - y0, y_ref - y0_ref)
    assert rel_fro(Wf - W0, W_ref - W0) <= BF16_TOL, rel_fro(Wf - W0, W_ref - W0)


def test_clip_4b_layer_shape():
    # d = 2560, f = 9728 (the Gram GEMMs at full width), 4 chunks of 256
    w = make_config("c3_4b_32k", T=1024)
    print(f"[clip 4b] d={w.d} f={w.f} T={w.T}", flush=True)
    y, Wf, y_ref, W_ref, W0 = _check(w, 256, 0, BF16_TOL, rel_fro)
    assert rel_fro(Wf - W0, W_ref - W0) <= BF16_TOL, rel_fro(Wf - W0, W_ref - W0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_clip_pages_threshold_4b(dtype):
    """The pages' threshold tau = 1e-5 at the 4B layer width, 16 chunks of 256 (T = 4096).

    Every chunk update (norm about 2e-2 here) is clipped to 1e-5, so each
    element of the state moves by about 1e-9 per chunk, below the fp32
    resolution of W itself (ulp 9e-10 at |W| = 0.01); the state is checked as
    W_final and as the accumulated update W_final - W_entry. The fast-weight
    part of y is below 1e-6 of y at this threshold, below fp32 (let alone
    bf16) resolution of y: on a 1024-token stream of this layer shape,
    rounding the oracle's exact y and y(eta=0) to fp32 already misses their
    difference by 0.12 (tests/test_precision_bounds.py), so y is checked as a
    whole.
    """
    import dataclasses
    w = make_config("c3_4b_32k", T=4096)
    if dtype == "f32":
        w = dataclasses.replace(w, dtype="f32")
    C, tau = 256, 1e-5
    print(f"[clip pages tau] {dtype} d={w.d} f={w.f} T={w.T} C={C} tau={tau}", flush=True)
    Z = oracle.gated_activation(w.x[0], w.W_up, w.W_gate)
    V = oracle.ntp_targets(w.ids[0], w.E_tgt)
    raw = [abs(w.eta) * np.linalg.norm(V[s:e].T @ Z[s:e]) for (s, e) in oracle.chunk_ranges(w.T, C)]
    assert min(raw) > 100 * tau  # every chunk is clipped, by a large factor
    del Z, V
    lay = Layer(w, C=C)
    ttt.ttt_set_clip(lay.h, tau)
    y, Wf = lay.forward_np()
    D = ttt.ttt_state_delta(lay.h, w.B).double().cpu().numpy()
    y_ref, W_ref = oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, C, w.eta, clip_tau=tau)
    W0 = w.W_down0.astype(np.float64)
    dn = np.linalg.norm(W_ref[0] - W0)
    assert dn <= len(raw) * tau * (1 + 1e-9)  # the applied updates have norm tau each
    metric, tol = (rel_fro, BF16_TOL) if dtype == "bf16" else (max_rel, F32_TOL)
    e_y, e_w, e_d = metric(y, y_ref), metric(Wf, W_ref), metric(D, W_ref - W0)
    # W_final itself is W0 + D rounded to fp32, which cannot hold an update this small to 3e-2: the rounding of
    # the exact result alone is about that large
    floor = rel_fro(W_ref.astype(np.float32).astype(np.float64) - W0, W_ref - W0)
    print(f"  |W_final - W0| = {dn:.3e}; y err {e_y:.2e}, W_final err {e_w:.2e}, D err {e_d:.2e} "
          f"(fp32 W_final - W0: {metric(Wf - W0, W_ref - W0):.2e}, its rounding floor {floor:.2e})", flush=True)
    assert e_y <= tol and e_w <= tol and e_d <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_clip_deterministic_and_switchable(dtype):
    d, f = (64, 128) if dtype == "f32" else (256, 256)
    w = make_inputs(d=d, f=f, B=2, T=900, C=64, eta=2e-3, dtype=dtype, vocab=77, e_std=1.0, seed=61)
    lay = Layer(w)
    y_plain, W_plain = lay.forward()
    y_plain, W_plain = y_plain.clone(), W_plain.clone()
    tau = _clip_threshold(w, 64)
    ttt.ttt_set_clip(lay.h, tau)
    ttt.ttt_reset(lay.h)
    y1, W1 = lay.forward()
    y1, W1 = y1.clone(), W1.clone()
    ttt.ttt_reset(lay.h)
    y2, W2 = lay.forward()
    assert torch.equal(y1, y2) and torch.equal(W1, W2)  # bitwise deterministic
    assert not torch.equal(W1, W_plain)
    # tau = +inf turns clipping off again: the unclipped result, bit for bit
    ttt.ttt_set_clip(lay.h, float("inf"))
    ttt.ttt_reset(lay.h)
    y3, W3 = lay.forward()
    assert torch.equal(y3, y_plain) and torch.equal(W3, W_plain)
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_set_clip(lay.h, -1.0)
    assert e.value.code == -7
