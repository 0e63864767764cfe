"""The CPU oracle against its pins (closed forms, autograd, library special cases, invariants)."""
import numpy as np
import pytest
import torch

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: getattr(p, "__name__", "pin"))
def test_oracle_pin(pin):
    pin(oracle.ttt_forward)


def test_final_state_columns_match_full_state():
    rng = np.random.default_rng(11)
    x, ids, E, Wu, Wg, W0 = pins.tiny_case(rng, d=7, f=12, B=1, T=19)
    _, W = oracle.ttt_forward(x, ids, E, Wu, Wg, W0, 4, 0.3)
    cols = [0, 5, 11, 3]
    Wc = oracle.final_state_columns(x[0], ids[0], E, Wu, Wg, W0, 4, 0.3, cols)
    ref = pins.block_causal_closed_form(x[0], ids[0], E, Wu, Wg, W0, 4, 0.3)[1][:, cols]
    assert np.max(np.abs(Wc - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.max(np.abs(Wc - W[0][:, cols])) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("T,C,t0,t1,block", [
    (37, 4, 0, 37, 8), (37, 4, 13, 29, 5), (37, 5, 20, 20, 3), (40, 8, 32, 40, 7), (23, 1, 9, 17, 4),
    (23, 30, 4, 11, 2), (50, 6, 49, 50, 16)])
def test_window_outputs_match_sequential_and_closed_form(T, C, t0, t1, block):
    # the window form against the sequential apply-then-update loop and against the block-causal closed form
    # (linear attention with a block mask, written in tests/pins.py), at windows that start inside a chunk,
    # on a chunk boundary, are empty, or hold the stream's last token
    rng = np.random.default_rng(T * 100 + t0)
    x, ids, E, Wu, Wg, W0 = pins.tiny_case(rng, d=7, f=12, B=1, T=T)
    y_seq, _ = oracle.ttt_forward(x, ids, E, Wu, Wg, W0, C, 0.3)
    y_cf = pins.block_causal_closed_form(x[0], ids[0], E, Wu, Wg, W0, C, 0.3)[0]
    yw = oracle.window_outputs(x[0], ids[0], E, Wu, Wg, W0, C, 0.3, t0, t1, block=block)
    assert yw.shape == (t1 - t0, 7)
    scale = max(np.max(np.abs(y_seq)), 1e-300)
    assert np.max(np.abs(yw - y_seq[0, t0:t1]), initial=0.0) <= 1e-12 * scale
    assert np.max(np.abs(yw - y_cf[t0:t1]), initial=0.0) <= 1e-12 * scale


def test_window_outputs_rejects_bad_window():
    rng = np.random.default_rng(3)
    x, ids, E, Wu, Wg, W0 = pins.tiny_case(rng, T=10)
    with pytest.raises(ValueError):
        oracle.window_outputs(x[0], ids[0], E, Wu, Wg, W0, 4, 0.3, 6, 5)
    with pytest.raises(ValueError):
        oracle.window_outputs(x[0], ids[0], E, Wu, Wg, W0, 4, 0.3, 0, 11)


def test_chunk_ranges():
    assert oracle.chunk_ranges(0, 4) == []
    assert oracle.chunk_ranges(10, 4) == [(0, 4), (4, 8), (8, 10)]
    assert oracle.chunk_ranges(8, 8) == [(0, 8)]
    assert oracle.chunk_ranges(3, 100) == [(0, 3)]
    with pytest.raises(ValueError):
        oracle.chunk_ranges(5, 0)


def test_empty_stream():
    rng = np.random.default_rng(0)
    x, ids, E, Wu, Wg, W0 = pins.tiny_case(rng, T=0)
    y, W = oracle.ttt_forward(x, ids, E, Wu, Wg, W0, 4, 0.5)
    assert y.shape == (1, 0, 6)
    assert np.array_equal(W[0], W0)


def test_silu_textbook_values():
    # SiLU(0) = 0; SiLU(ln 3) = ln 3 * 3/4 (sigmoid(ln 3) = 3/4); odd part SiLU(g) - SiLU(-g) = g
    g = np.array([0.0, np.log(3.0), -np.log(3.0), 2.5])
    s = oracle.silu(g)
    assert s[0] == 0.0
    assert abs(s[1] - 0.75 * np.log(3.0)) < 1e-15
    assert abs(s[2] + 0.25 * np.log(3.0)) < 1e-15
    assert abs((oracle.silu(2.5) - oracle.silu(-2.5)) - 2.5) < 1e-14
    assert np.allclose(s, torch.nn.functional.silu(torch.from_numpy(g)).numpy(), rtol=1e-15, atol=0)
