"""The allocation-free forward (ttt_forward_chunked_noalloc) against ttt_forward_chunked, through the C ABI.

Two calls in a row on one handle, the second with a smaller input (fewer
sequences, a shorter block): each must equal what ttt_forward_chunked gives on
the same input from the same state, bit for bit (the same kernels run on a
workspace at another address), and so also within the parity bar against the
oracle. The handle that makes the allocation-free calls never grows a
scratch buffer of its own.
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as ttt
import oracle
from synth import make_inputs
from tests.gpu_util import Layer, max_rel, rel_fro

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_forward_on_two_calls(dtype):
    d, f = (256, 512) if dtype == "bf16" else (64, 256)
    w = make_inputs(d=d, f=f, B=2, T=3000, C=128, eta=2e-3, dtype=dtype, vocab=300, e_std=1.0, seed=71)
    print(f"[noalloc] {dtype} d={d} f={f} B={w.B} T={w.T}, then B=1 T=1000", flush=True)
    ref = Layer(w)
    na = Layer(w)
    ws0 = ttt.ttt_workspace_bytes(na.h)
    # call 1: the full input
    y_ref, W_ref = ref.forward()
    y = torch.empty_like(y_ref)
    Wf = torch.empty_like(W_ref)
    ttt.ttt_forward_chunked_noalloc(na.h, na.x, na.ids, na.E, y, Wf)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(Wf, W_ref)
    # call 2: a smaller input (one sequence, 1000 tokens) from reset states
    ttt.ttt_reset(ref.h)
    ttt.ttt_reset(na.h)
    x2, ids2 = na.x[:1, :1000].contiguous(), na.ids[:1, :1001].contiguous()
    y2_ref, W2_ref = ttt.ttt_forward_chunked(ref.h, x2, ids2, ref.E, want_W_final=True)
    y2 = torch.empty_like(y2_ref)
    W2 = torch.empty_like(W2_ref)
    ttt.ttt_forward_chunked_noalloc(na.h, x2, ids2, na.E, y2, W2)
    torch.cuda.synchronize()
    assert torch.equal(y2, y2_ref) and torch.equal(W2, W2_ref)
    assert ttt.ttt_workspace_bytes(na.h) == ws0  # no scratch of the handle's own
    # and the parity bar against the oracle on the second call
    y_o, W_o = oracle.ttt_forward(w.x[:1, :1000], w.ids[:1, :1001], w.E_tgt, w.W_up, w.W_gate, w.W_down0, w.C,
                                  w.eta)
    metric, tol = (rel_fro, 3e-2) if dtype == "bf16" else (max_rel, 1e-4)
    assert metric(y2.double().cpu().numpy(), y_o) <= tol
    assert metric(W2.double().cpu().numpy(), W_o) <= tol
    ttt.ttt_destroy(ref.h)
    ttt.ttt_destroy(na.h)


def test_noalloc_rejects_a_call_beyond_the_workspace():
    w = make_inputs(d=256, f=512, B=1, T=256, C=128, eta=2e-3, dtype="bf16", vocab=50, e_std=1.0, seed=72)
    lay = Layer(w)
    ws0 = ttt.ttt_workspace_bytes(lay.h)
    # 65536 tokens need Z and eta*Z^T alone of 2 x 65536 x 512 x 2 bytes = 128 MiB, more than the 64 MiB workspace;
    # the size check fails before any device work, so the inputs are never read
    T = 65536
    x = torch.zeros((1, T, 256), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((1, T + 1), dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_forward_chunked_noalloc(lay.h, x, ids, lay.E, y)
    assert e.value.code == -2
    assert "workspace" in ttt.ttt_last_error()
    assert ttt.ttt_workspace_bytes(lay.h) == ws0
    ttt.ttt_destroy(lay.h)
