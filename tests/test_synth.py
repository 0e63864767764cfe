"""Seeded input generators: determinism, shapes, distributions, bf16 rounding."""
import numpy as np
import torch

from synth import CONFIGS, bf16_bits, bf16_round, make_config, make_inputs


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-6, 6, 100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3e38], dtype=np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(a), ref)
    r = bf16_round(a)
    assert np.array_equal(torch.from_numpy(r).to(torch.bfloat16).float().numpy(), r)


def test_make_inputs_deterministic_and_shaped():
    kw = dict(d=64, f=128, B=2, T=40, C=8, eta=1e-2, dtype="bf16", vocab=100, e_std=0.02, seed=3)
    a = make_inputs(**kw)
    b = make_inputs(**kw)
    for k in ("W_up", "W_gate", "W_down0", "E_tgt", "x", "ids"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    assert a.W_up.shape == (128, 64) and a.W_down0.shape == (64, 128)
    assert a.x.shape == (2, 40, 64) and a.ids.shape == (2, 41) and a.ids.dtype == np.int32
    assert a.ids.min() >= 0 and a.ids.max() < 100
    assert np.array_equal(bf16_round(a.x), a.x)


def test_rmsnorm_rows():
    w = make_inputs(d=256, f=64, B=1, T=16, C=8, eta=0.0, dtype="f32", vocab=10, e_std=1.0,
                    x_kind="rmsnorm", seed=1)
    rms = np.sqrt(np.mean(w.x.astype(np.float64) ** 2, axis=-1))
    assert np.allclose(rms, 1.0, atol=1e-5)


def test_config_table():
    assert set(CONFIGS) == {"c1_tiny_f32", "c2_1k4k_b4", "c3_4b_32k", "c4_4b_128k", "c5_4b_stack36"}
    w = make_config("c1_tiny_f32")
    assert (w.d, w.f, w.B, w.T, w.C, w.eta, w.dtype, w.vocab) == (64, 256, 1, 1024, 128, 0.01, "f32", 512)
    assert abs(np.std(w.W_up) - 1 / 8) < 0.01 and abs(np.std(w.W_down0) - 1 / 16) < 0.005
    assert abs(np.std(w.E_tgt) - 1.0) < 0.05
