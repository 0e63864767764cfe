"""GPU parity for the general target V^ = Conv1D(X0) W_target (paperlayer
sec. 3 "LM-Aligned Objective"; iplexlaw sec. 4 and sec. 6), against the oracle
with the same taps, projection and chunk-boundary padding.

E_tgt is then the token-embedding table X0. Cases cover chunks shorter than
the kernel (taps cut by the chunk boundary), per-token chunks, one chunk,
clipping together with the general target, and the 4B layer shape. With one
tap of weight 1 and W_target = I the result is the next-token path's, bit for
bit. Tolerances as in the other parity tests.
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as ttt
import oracle
from synth import make_config, make_inputs, make_target_conv
from tests.gpu_util import Layer, dev, max_rel, rel_fro

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 3e-2


def _layer(w, cw, Wt, C=None, eta=None, G=0, clip=0.0):
    lay = Layer(w, C=C, eta=eta, G=G)
    ttt.ttt_set_target_conv(lay.h, dev(cw, lay.dt), dev(Wt, lay.dt))
    if clip:
        ttt.ttt_set_clip(lay.h, clip)
    return lay


def _oracle(w, cw, Wt, C, eta=None, clip=None):
    return oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, C, w.eta if eta is None else eta,
                              clip_tau=clip, conv_w=cw, W_target=Wt)


FP32_CASES = [  # (T, C, B, K)
    (1000, 100, 2, 5),
    (600, 3, 1, 5),     # chunks shorter than the kernel
    (640, 1, 1, 5),     # per-token chunks: only the next token is reachable
    (500, 600, 1, 5),   # one chunk
    (900, 64, 1, 2),
]


@pytest.mark.parametrize("T,C,B,K", FP32_CASES)
def test_target_fp32(T, C, B, K):
    w = make_inputs(d=64, f=192, B=B, T=T, C=C, eta=0.02, dtype="f32", vocab=97, e_std=1.0, seed=70 + T)
    cw, Wt = make_target_conv(64, K, "f32", seed=T)
    print(f"[target fp32] T={T} C={C} B={B} K={K}", flush=True)
    y, Wf = _layer(w, cw, Wt, C=C).forward_np()
    y_ref, W_ref = _oracle(w, cw, Wt, C)
    assert max_rel(y, y_ref) <= F32_TOL, max_rel(y, y_ref)
    assert max_rel(Wf, W_ref) <= F32_TOL, max_rel(Wf, W_ref)


BF16_CASES = [  # (T, C, B, K)
    (3000, 128, 2, 5),
    (2500, 24, 1, 5),
    (1500, 3, 1, 5),
    (1500, 1, 1, 5),
    (4096, 512, 1, 5),
    (700, 1024, 1, 5),
]


@pytest.mark.parametrize("T,C,B,K", BF16_CASES)
def test_target_bf16(T, C, B, K):
    w = make_inputs(d=256, f=512, B=B, T=T, C=C, eta=1e-3, dtype="bf16", vocab=301, e_std=1.0, seed=80 + T + C)
    cw, Wt = make_target_conv(256, K, "bf16", seed=T + C)
    print(f"[target bf16] T={T} C={C} B={B} K={K}", flush=True)
    y, Wf = _layer(w, cw, Wt, C=C).forward_np()
    y0, _ = _layer(w, cw, Wt, C=C, eta=0.0).forward_np()
    y_ref, W_ref = _oracle(w, cw, Wt, C)
    y0_ref, _ = _oracle(w, cw, Wt, C, eta=0.0)
    W0 = w.W_down0.astype(np.float64)
    assert rel_fro(y, y_ref) <= BF16_TOL, rel_fro(y, y_ref)
    assert rel_fro(Wf, W_ref) <= BF16_TOL, rel_fro(Wf, W_ref)
    assert rel_fro(y - y0, y_ref - y0_ref) <= BF16_TOL, rel_fro(y - y0, y_ref - y0_ref)
    assert rel_fro(Wf - W0, W_ref - W0) <= BF16_TOL, rel_fro(Wf - W0, W_ref - W0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_target_with_clipping(dtype):
    d, f, eta = (64, 192, 0.02) if dtype == "f32" else (256, 512, 1e-3)
    w = make_inputs(d=d, f=f, B=2, T=1200, C=100, eta=eta, dtype=dtype, vocab=150, e_std=1.0, seed=91)
    cw, Wt = make_target_conv(d, 5, dtype, seed=9)
    _, W_raw = _oracle(w, cw, Wt, 100)
    tau = 0.2 * float(np.linalg.norm(W_raw[0] - w.W_down0)) / np.sqrt(12)  # below the typical chunk norm
    y, Wf = _layer(w, cw, Wt, C=100, clip=tau).forward_np()
    y_ref, W_ref = _oracle(w, cw, Wt, 100, clip=tau)
    metric, tol = (max_rel, F32_TOL) if dtype == "f32" else (rel_fro, BF16_TOL)
    assert np.linalg.norm(W_ref - W_raw) > 0.01 * np.linalg.norm(W_raw - w.W_down0)
    assert metric(y, y_ref) <= tol, metric(y, y_ref)
    assert metric(Wf, W_ref) <= tol, metric(Wf, W_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_tap_identity_equals_next_token(dtype):
    d, f = (64, 128) if dtype == "f32" else (256, 256)
    w = make_inputs(d=d, f=f, B=2, T=900, C=64, eta=2e-3, dtype=dtype, vocab=77, e_std=1.0, seed=93)
    lay = Layer(w)
    y0, W0 = lay.forward()
    y0, W0 = y0.clone(), W0.clone()
    ttt.ttt_set_target_conv(lay.h, torch.ones((1, d), dtype=lay.dt, device="cuda"),
                            torch.eye(d, dtype=lay.dt, device="cuda"))
    ttt.ttt_reset(lay.h)
    y1, W1 = lay.forward()
    assert torch.equal(y1, y0) and torch.equal(W1, W0)
    ttt.ttt_set_target_conv(lay.h, None)  # back to the next-token rows
    ttt.ttt_reset(lay.h)
    y2, W2 = lay.forward()
    assert torch.equal(y2, y0) and torch.equal(W2, W0)


def test_target_4b_layer_shape():
    w = make_config("c3_4b_32k", T=1024)
    cw, Wt = make_target_conv(w.d, 5, "bf16", seed=4)
    print(f"[target 4b] d={w.d} f={w.f} T={w.T}", flush=True)
    y, Wf = _layer(w, cw, Wt, C=256).forward_np()
    y_ref, W_ref = _oracle(w, cw, Wt, 256)
    W0 = w.W_down0.astype(np.float64)
    assert rel_fro(y, y_ref) <= BF16_TOL, rel_fro(y, y_ref)
    assert rel_fro(Wf - W0, W_ref - W0) <= BF16_TOL, rel_fro(Wf - W0, W_ref - W0)
