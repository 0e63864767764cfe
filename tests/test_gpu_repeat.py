"""Repeated forwards at the 4B layer width must agree bit for bit.

A fault that depends on timing (an LDS write landing after a read, a store
racing a later write) shows as a run-to-run difference, which the tolerance
checks of the parity tests can miss when few elements are hit. Each mode runs
the same call three times from a reset state, at d = 2560, f = 9728 and 4096
tokens: 4.75 rounds of up/gate tiles, a whole round and a half-tile round of
the update, 160 output tiles, and, with the general target or clipping, the
target GEMM and the chunk Grams; packed documents of ragged lengths run as
one launch sequence over a sequence table.
"""
from __future__ import annotations

import pytest
import torch

import chunk_wise_weight_amd as ttt
from synth import make_inputs, make_target_conv
from tests.gpu_util import Layer, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4b():
    return make_inputs(d=2560, f=9728, B=1, T=4096, C=256, eta=1e-3, dtype="bf16", vocab=512, e_std=1.0, seed=123)


@pytest.mark.parametrize("mode", ["plain", "target", "clip", "docs"])
def test_repeat_bitwise_4b_width(w4b, mode):
    lay = Layer(w4b)
    if mode == "target":
        cw, Wt = make_target_conv(w4b.d, 5, "bf16", seed=5)
        ttt.ttt_set_target_conv(lay.h, dev(cw, lay.dt), dev(Wt, lay.dt))
    elif mode == "clip":
        ttt.ttt_set_clip(lay.h, 1e-5)  # the pages' threshold
    runs = []
    for _ in range(3):
        ttt.ttt_reset(lay.h)
        if mode == "docs":  # ragged packed documents: one launch sequence with a sequence table
            y, Wf = ttt.ttt_forward_docs(lay.h, lay.x, lay.ids, lay.E, [[700, 1900, 2100, 3333]], want_W_final=True)
            torch.cuda.synchronize()
        else:
            y, Wf = lay.forward()
        runs.append((y.clone(), Wf.clone()))
    y0, W0 = runs[0]
    assert torch.isfinite(y0.float()).all() and torch.isfinite(W0).all()
    assert float(y0.float().abs().max()) > 0
    for y, Wf in runs[1:]:
        dy = int((y != y0).sum())
        dW = int((Wf != W0).sum())
        assert dy == 0 and dW == 0, f"{mode}: {dy} elements of y and {dW} of W_final differ between runs"
    ttt.ttt_destroy(lay.h)
