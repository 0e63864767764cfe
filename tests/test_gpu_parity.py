"""GPU parity: the HIP path against the CPU oracle, element by element.

Tolerances: fp32 path <= 1e-4 max-relative (max|a-r| / max|r|) on y and the
final state; bf16 path <= 3e-2 relative Frobenius. Because the fast-weight
term can be small next to the static part, the bf16 checks also compare the
TTT contributions themselves: y - y(eta=0) and W_final - W_entry.
Sizes span several 256-tiles, several snapshot groups and ragged tails, and
use a learning rate large enough that the update term is comparable to the
static one.
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as ttt
import oracle
from synth import make_config, make_inputs
from tests.gpu_util import Layer, dev, max_rel, rel_fro

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 3e-2


def _oracle(w, C=None, eta=None):
    return oracle.ttt_forward(w.x, w.ids, w.E_tgt, w.W_up, w.W_gate, w.W_down0, C or w.C,
                              w.eta if eta is None else eta)


def test_c1_tiny_fp32_full_config():
    w = make_config("c1_tiny_f32")
    print(f"[c1] d={w.d} f={w.f} T={w.T} C={w.C}", flush=True)
    y, Wf = Layer(w).forward_np()
    y_ref, W_ref = _oracle(w)
    assert max_rel(y, y_ref) <= F32_TOL
    assert max_rel(Wf, W_ref) <= F32_TOL
    # the update is several times W_down0 here, so the scan terms dominate
    assert np.linalg.norm(W_ref[0] - w.W_down0) > np.linalg.norm(w.W_down0)


FP32_CASES = [  # (T, C, G, B)
    (1000, 100, 0, 2),   # ragged chunks, group starts inside 16-token steps
    (777, 128, 0, 1),    # ragged last chunk
    (640, 1, 0, 1),      # per-token updates
    (500, 600, 0, 1),    # C >= T: one chunk
    (2048, 64, 2, 2),    # small groups: many snapshots
    (1500, 24, 0, 1),    # C < 64, not a power of two
    (1300, 8, 16, 1),    # group of 128 tokens
]


@pytest.mark.parametrize("T,C,G,B", FP32_CASES)
def test_fp32_variants(T, C, G, B):
    w = make_inputs(d=64, f=192, B=B, T=T, C=C, eta=0.02, dtype="f32", vocab=97, e_std=1.0, seed=10 + T)
    print(f"[fp32] T={T} C={C} G={G} B={B}", flush=True)
    y, Wf = Layer(w, G=G).forward_np()
    y_ref, W_ref = _oracle(w)
    assert max_rel(y, y_ref) <= F32_TOL, max_rel(y, y_ref)
    assert max_rel(Wf, W_ref) <= F32_TOL, max_rel(Wf, W_ref)


BF16_CASES = [  # (T, C, G, B)
    (3000, 128, 0, 2),
    (3000, 256, 0, 1),
    (3000, 100, 0, 1),   # chunks of 100 cross the 64-token slabs; groups of 1600
    (1500, 1, 0, 1),     # per-token updates, causal within-group term
    (700, 1024, 0, 1),   # one chunk
    (4096, 128, 2, 1),   # groups of 256 tokens
    (2500, 24, 0, 1),    # C < 64
    (2100, 512, 0, 1),   # C = 512: one chunk per group pair
]


@pytest.mark.parametrize("T,C,G,B", BF16_CASES)
def test_bf16_variants(T, C, G, B):
    w = make_inputs(d=256, f=512, B=B, T=T, C=C, eta=1e-3, dtype="bf16", vocab=301, e_std=1.0, seed=20 + T + C)
    print(f"[bf16] T={T} C={C} G={G} B={B}", flush=True)
    lay = Layer(w, G=G)
    y, Wf = lay.forward_np()
    lay0 = Layer(w, G=G, eta=0.0)
    y0, Wf0 = lay0.forward_np()
    y_ref, W_ref = _oracle(w)
    y0_ref, _ = _oracle(w, eta=0.0)
    W0 = w.W_down0.astype(np.float64)
    assert rel_fro(y, y_ref) <= BF16_TOL, rel_fro(y, y_ref)
    assert rel_fro(Wf, W_ref) <= BF16_TOL, rel_fro(Wf, W_ref)
    assert rel_fro(y - y0, y_ref - y0_ref) <= BF16_TOL, rel_fro(y - y0, y_ref - y0_ref)
    assert rel_fro(Wf - W0, W_ref - W0) <= BF16_TOL, rel_fro(Wf - W0, W_ref - W0)
    # eta = 0 leaves the state untouched, bit for bit
    assert np.array_equal(Wf0, np.broadcast_to(W0, Wf0.shape))


SHORT_4B_CASES = [  # (T, C, G, B) at d = 2560, f = 9728
    (64, 64, 0, 1),     # one slab
    (200, 64, 2, 1),    # odd stage count, groups of 128 tokens
    (333, 64, 1, 2),    # a snapshot every 64 tokens; 760 tiles, all on the 256 x 256 shape
    (333, 100, 0, 1),   # 380 tiles, one group: whole round and half-tile round
    (1150, 64, 2, 1),   # 380 tiles, 9 groups of 128 tokens in both rounds, ragged tail
]


@pytest.mark.parametrize("T,C,G,B", SHORT_4B_CASES)
def test_bf16_4b_shape_short_streams(T, C, G, B):
    # At the 4B layer width the state has 380 tiles per sequence, so the update
    # runs its 256 x 256 kernel (with the L2 prefetch two slabs ahead, clamped
    # to the last slab) on streams of only a few slabs.
    w = make_inputs(d=2560, f=9728, B=B, T=T, C=C, eta=1e-3, dtype="bf16", vocab=509, e_std=0.5, seed=70 + T + G)
    print(f"[bf16 4b short] T={T} C={C} G={G} B={B}", flush=True)
    y, Wf = Layer(w, G=G).forward_np()
    y0, _ = Layer(w, G=G, eta=0.0).forward_np()
    y_ref, W_ref = _oracle(w)
    y0_ref, _ = _oracle(w, eta=0.0)
    W0 = w.W_down0.astype(np.float64)
    assert rel_fro(y, y_ref) <= BF16_TOL, rel_fro(y, y_ref)
    assert rel_fro(y - y0, y_ref - y0_ref) <= BF16_TOL, rel_fro(y - y0, y_ref - y0_ref)
    assert rel_fro(Wf - W0, W_ref - W0) <= BF16_TOL, rel_fro(Wf - W0, W_ref - W0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_static_and_empty(dtype):
    d, f = (64, 128) if dtype == "f32" else (256, 256)
    w = make_inputs(d=d, f=f, B=2, T=300, C=64, eta=0.0, dtype=dtype, vocab=50, e_std=1.0, seed=5)
    lay = Layer(w)
    y, Wf = lay.forward_np()
    y_ref, _ = _oracle(w)
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    metric = max_rel if dtype == "f32" else rel_fro
    assert metric(y, y_ref) <= tol
    # T = 0: nothing to do, final state returned unchanged
    x0 = torch.empty((2, 0, d), dtype=lay.dt, device="cuda")
    ids0 = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    y_e, W_e = ttt.ttt_forward_chunked(lay.h, x0, ids0, lay.E, want_W_final=True)
    torch.cuda.synchronize()
    assert y_e.shape == (2, 0, d)
    assert np.array_equal(W_e.double().cpu().numpy(), np.broadcast_to(w.W_down0, (2, d, f)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reset_segments_batch_determinism(dtype):
    d, f = (64, 128) if dtype == "f32" else (256, 512)
    C, T1, T2 = 128, 768, 1000
    w = make_inputs(d=d, f=f, B=3, T=T1 + T2, C=C, eta=2e-3, dtype=dtype, vocab=200, e_std=1.0, seed=7)
    lay = Layer(w)
    y_full, W_full = lay.forward()
    y_full, W_full = y_full.clone(), W_full.clone()
    # determinism: a second run from a reset state is bitwise identical
    ttt.ttt_reset(lay.h)
    y_b, W_b = lay.forward()
    assert torch.equal(y_b, y_full) and torch.equal(W_b, W_full)
    # reset restores W_down0 bit for bit (fp32 image of the given W_down0)
    ttt.ttt_reset(lay.h)
    _, W_r = ttt.ttt_forward_chunked(lay.h, lay.x[:, :0].contiguous(), lay.ids[:, :1].contiguous(), lay.E,
                                     want_W_final=True)
    torch.cuda.synchronize()
    assert np.array_equal(W_r.double().cpu().numpy(), np.broadcast_to(w.W_down0, W_r.shape))
    # resume: T1 (a multiple of C) then T2 tokens equals one call (the split moves group boundaries,
    # so the bf16 path agrees to rounding, the fp32 path to fp32 rounding)
    ya, Wa = lay.forward(lay.x[:, :T1].contiguous(), lay.ids[:, :T1 + 1].contiguous())
    ya = ya.clone()
    yb, Wb = lay.forward(lay.x[:, T1:].contiguous(), lay.ids[:, T1:].contiguous())
    y2 = torch.cat([ya, yb], dim=1).double().cpu().numpy()
    tol, metric = (F32_TOL, max_rel) if dtype == "f32" else (BF16_TOL, rel_fro)
    assert metric(y2, y_full.double().cpu().numpy()) <= tol
    assert metric(Wb.double().cpu().numpy(), W_full.double().cpu().numpy()) <= tol
    # per-sequence reset: only sequence 1 returns to W_down0
    ttt.ttt_reset(lay.h, 1)
    _, W_p = ttt.ttt_forward_chunked(lay.h, lay.x[:, :0].contiguous(), lay.ids[:, :1].contiguous(), lay.E,
                                     want_W_final=True)
    torch.cuda.synchronize()
    assert torch.equal(W_p[0], Wb[0]) and torch.equal(W_p[2], Wb[2])
    assert np.array_equal(W_p[1].double().cpu().numpy(), w.W_down0)
    # batch independence: sequence 2 alone (fresh state) gives the same bits as inside the batch
    ttt.ttt_reset(lay.h)
    y1, W1 = ttt.ttt_forward_chunked(lay.h, lay.x[2:3].contiguous(), lay.ids[2:3].contiguous(), lay.E,
                                     want_W_final=True)
    torch.cuda.synchronize()
    assert torch.equal(y1[0], y_full[2]) and torch.equal(W1[0], W_full[2])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_causality_bitwise(dtype):
    d, f = (64, 128) if dtype == "f32" else (256, 256)
    C, T = 128, 1536
    w = make_inputs(d=d, f=f, B=1, T=T, C=C, eta=2e-3, dtype=dtype, vocab=100, e_std=1.0, seed=9)
    lay = Layer(w)
    y0, _ = lay.forward()
    y0 = y0.clone()
    rng = np.random.default_rng(0)
    for i in (0, 3, 7, 10):
        end = (i + 1) * C
        ttt.ttt_reset(lay.h)
        x2 = lay.x.clone()
        x2[:, end:] = dev(rng.standard_normal((1, T - end, d)).astype(np.float32), lay.dt)
        ids2 = lay.ids.clone()
        ids2[:, end + 1:] = torch.from_numpy(rng.integers(0, 100, (1, T - end))).to(torch.int32).cuda()
        y1, _ = lay.forward(x2, ids2)
        assert torch.equal(y1[:, :end], y0[:, :end]), f"chunk {i}: later tokens changed earlier outputs"
        ttt.ttt_reset(lay.h)
    # the one-token shift: ids[(i+1)C] reaches chunk i+1's outputs
    ids3 = lay.ids.clone()
    ids3[0, 2 * C] = (ids3[0, 2 * C] + 1) % 100
    ttt.ttt_reset(lay.h)
    y3, _ = lay.forward(lay.x, ids3)
    assert torch.equal(y3[:, :2 * C], y0[:, :2 * C])
    assert not torch.equal(y3[:, 2 * C:3 * C], y0[:, 2 * C:3 * C])


def test_out_of_range_ids_zero_targets():
    w = make_inputs(d=256, f=256, B=1, T=600, C=100, eta=1e-3, dtype="bf16", vocab=64, e_std=1.0, seed=3)
    w.ids[0, ::3] = -1
    w.ids[0, 1::7] = 64 + 5
    lay = Layer(w)
    y, Wf = lay.forward_np()
    y_ref, W_ref = _oracle(w)
    W0 = w.W_down0.astype(np.float64)
    assert rel_fro(y, y_ref) <= BF16_TOL
    assert rel_fro(Wf - W0, W_ref - W0) <= BF16_TOL


TINY_CASES = [  # (T, C, B): streams shorter than one 8-token stage, a ragged 33 with chunks of 1, 4 and 16
    (1, 1, 1),
    (1, 256, 2),
    (7, 4, 1),
    (33, 1, 1),
    (33, 4, 2),
    (33, 16, 1),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,C,B", TINY_CASES)
def test_tiny_streams(dtype, T, C, B):
    # A single token only updates the state (its output uses the entry weight); a few tokens exercise the
    # ragged first slab of every kernel, the clamped L2 prefetch and the first snapshot alone.
    d, f = (64, 128) if dtype == "f32" else (256, 512)
    w = make_inputs(d=d, f=f, B=B, T=T, C=C, eta=0.05, dtype=dtype, vocab=31, e_std=1.0, seed=900 + 10 * T + C)
    print(f"[tiny] {dtype} T={T} C={C} B={B}", flush=True)
    y, Wf = Layer(w).forward_np()
    y_ref, W_ref = _oracle(w)
    W0 = w.W_down0.astype(np.float64)
    metric, tol = (max_rel, F32_TOL) if dtype == "f32" else (rel_fro, BF16_TOL)
    assert metric(y, y_ref) <= tol, metric(y, y_ref)
    assert metric(Wf, W_ref) <= tol, metric(Wf, W_ref)
    assert metric(Wf - W0, W_ref - W0) <= tol, metric(Wf - W0, W_ref - W0)
