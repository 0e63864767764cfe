"""What the output format itself can resolve of the fast-weight part of y.

These are arithmetic facts about the oracle's exact (fp64) results, no GPU
involved. They fix which parity checks on y - y(eta=0) are meaningful:
  * at the pages' clipping threshold tau = 1e-5 on the 4B layer, the
    fast-weight part of y is below 1e-6 of y, and merely rounding the exact y
    and y(eta=0) to fp32 misses their difference by more than 3e-2;
  * at the 1k/4k workload (d = 1024, f = 4096, 8192 tokens, C = 256) the
    fast-weight part in the last snapshot group is 7% of y, and rounding the
    exact y and y(eta=0) to bf16 misses their difference by more than 3e-2.
So no implementation that returns y in those formats can meet 3e-2 on the
difference there; the GPU tests check the state (W_final - W_entry) at tau =
1e-5, and the difference on fp32 y at the 1k/4k workload.
"""
import numpy as np

import oracle
from synth import make_config, make_inputs
from synth.workloads import bf16_round
from tests.gpu_util import rel_fro


def _fp32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def _bf16(a):
    return bf16_round(np.asarray(a, dtype=np.float64).astype(np.float32)).astype(np.float64)


def test_pages_tau_fast_weight_part_below_fp32_resolution():
    # the 4B layer recipe (d = 2560, f = 9728, RMS-normalised x, eta = 1e-3, target rows N(0, 0.02^2)) on a
    # 1024-token stream; a 4096-row target table stands in for the 151936-row one, whose rows are drawn alike
    w = make_inputs(d=2560, f=9728, B=1, T=1024, C=256, eta=1e-3, dtype="bf16", vocab=4096, e_std=0.02,
                    x_kind="rmsnorm", seed=3)
    C, tau = 256, 1e-5
    y, W = oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, C, w.eta, clip_tau=tau)
    y0, _ = oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, C, 0.0)
    part = np.linalg.norm(y - y0) / np.linalg.norm(y)
    assert part < 1e-6
    assert rel_fro(_fp32(y) - _fp32(y0), y - y0) > 3e-2
    # the state itself still carries the update at full relative precision in fp64 terms
    D = W[0] - w.W_down0.astype(np.float64)
    assert 0 < np.linalg.norm(D) <= 4 * tau * (1 + 1e-9)  # four chunk updates of norm tau


def test_bf16_y_blurs_fast_weight_part_on_1k4k_workload():
    w = make_config("c2_1k4k_b4", B=1)
    C, L = 256, 1024
    t0, t1 = 7 * L + C, 8 * L  # chunks 1-3 of the last snapshot group
    y = oracle.window_outputs(w.x[0], w.ids[0], w.E_tgt, w.W_up, w.W_gate, w.W_down0, C, w.eta, t0, t1)
    y0 = oracle.gated_activation(w.x[0, t0:t1], w.W_up, w.W_gate) @ w.W_down0.astype(np.float64).T
    part = np.linalg.norm(y - y0) / np.linalg.norm(y)
    assert 0.05 < part < 0.1
    assert rel_fro(_bf16(y) - _bf16(y0), y - y0) > 3e-2
    assert rel_fro(_fp32(y) - _fp32(y0), y - y0) < 1e-5
