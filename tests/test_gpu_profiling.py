"""Per-phase device timing: the event ring behind ttt_phase_times (the mean
per forward call over the calls since the previous read)."""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as ttt
from synth import make_inputs
from tests.gpu_util import Layer

pytestmark = pytest.mark.gpu


def _layer():
    w = make_inputs(d=256, f=512, B=1, T=2048, C=64, eta=1e-3, dtype="bf16", vocab=300, e_std=0.5, seed=91)
    lay = Layer(w)
    ttt.ttt_set_profiling(lay.h, True)
    return lay


def test_phase_times_window_and_repeat():
    print("[profiling] window of 3 calls, repeat read", flush=True)
    lay = _layer()
    with pytest.raises(ttt.TTTError):
        ttt.ttt_phase_times(lay.h)  # no profiled call yet
    for _ in range(3):
        lay.forward()
    ph = ttt.ttt_phase_times(lay.h)
    assert len(ph) == len(ttt.PHASES)
    assert all(v >= 0.0 for v in ph)
    names = dict(zip(ttt.PHASES, ph))
    assert names["up_gate_swiglu"] > 0.0 and names["update_snapshots"] > 0.0 and names["output"] > 0.0
    assert names["clip_factors"] < 0.05  # clipping is off: two events with nothing between them
    # no call since the previous read: the same figures again
    assert ttt.ttt_phase_times(lay.h) == ph
    ttt.ttt_destroy(lay.h)


def test_phase_times_many_calls_between_reads():
    # more launch sequences than the ring's 16 event sets: the oldest are folded into running sums, and the
    # figures stay the mean per call
    print("[profiling] 40 calls between reads, then one docs call of 20 documents", flush=True)
    lay = _layer()
    for _ in range(4):
        lay.forward()
    short = np.array(ttt.ttt_phase_times(lay.h))
    for _ in range(40):
        ttt.ttt_forward_chunked(lay.h, lay.x, lay.ids, lay.E)
    torch.cuda.synchronize()
    many = np.array(ttt.ttt_phase_times(lay.h))
    i = ttt.PHASES.index("up_gate_swiglu")
    assert 0.5 * short[i] < many[i] < 2.0 * short[i] + 0.05
    # one call of 20 documents
    ttt.ttt_reset(lay.h)
    starts = [[100 * k for k in range(1, 20)]]
    ttt.ttt_forward_docs(lay.h, lay.x, lay.ids, lay.E, starts)
    torch.cuda.synchronize()
    docs = np.array(ttt.ttt_phase_times(lay.h))
    assert docs[i] > 0.0 and np.all(docs >= 0.0)
    ttt.ttt_destroy(lay.h)


def test_phase_times_docs_sum_their_documents():
    print("[profiling] docs call against plain call", flush=True)
    lay = _layer()
    lay.forward()
    plain = np.array(ttt.ttt_phase_times(lay.h))
    ttt.ttt_reset(lay.h)
    ttt.ttt_forward_docs(lay.h, lay.x, lay.ids, lay.E, [[512, 1024, 1536]])
    torch.cuda.synchronize()
    docs = np.array(ttt.ttt_phase_times(lay.h))
    # four launch sequences of a quarter of the tokens each, summed into one call's figures:
    # the up/gate phase covers the same tokens, so it stays within a few launches' overhead
    i = ttt.PHASES.index("up_gate_swiglu")
    assert docs[i] > 0.5 * plain[i]
    assert docs[i] < 4.0 * plain[i] + 0.2
    ttt.ttt_destroy(lay.h)
