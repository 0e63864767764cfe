"""Seeded synthetic workloads shaped like the pages' In-Place TTT efficiency runs.

The pages measure prefill of a continual-pretrained Qwen3-4B-Base (d_model 2560,
d_ff 9728, SwiGLU) at 8k-128k tokens, batch 1 (paperlayer.ai summary, App. C.2;
iplexlaw.co.kr walkthrough, sec. 7.5, Fig. 4). No checkpoint or dataset is
available here, so every tensor is drawn from a seeded generator with the
distributions listed per workload below.

Draw order for one layer is fixed: W_up, W_gate, W_down0, E_tgt, x, ids.
Values are drawn in fp32 and, for bf16 workloads, rounded once to bf16 with
round-to-nearest-even. Both the oracle and the GPU path consume the rounded
values, so they see identical inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even. Finite inputs only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (RNE), returned as fp32."""
    return (bf16_bits(a).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One layer's inputs plus the method's parameters.

    Layouts (row-major): W_up, W_gate [f][d]; W_down0 [d][f]; E_tgt [vocab][d];
    x [B][T][d]; ids [B][T+1] int32 (ids[b][T] is the look-ahead token).
    Float arrays are fp32 holding exactly representable values of `dtype`.
    """

    name: str
    d: int
    f: int
    B: int
    T: int
    C: int
    eta: float
    dtype: str  # "f32" or "bf16"
    vocab: int
    W_up: np.ndarray
    W_gate: np.ndarray
    W_down0: np.ndarray
    E_tgt: np.ndarray
    x: np.ndarray
    ids: np.ndarray
    meta: Dict[str, object] = field(default_factory=dict)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def make_inputs(
    *,
    d: int,
    f: int,
    B: int,
    T: int,
    C: int,
    eta: float,
    dtype: str,
    vocab: int,
    e_std: float,
    x_kind: str = "normal",
    seed=0,
    name: str = "custom",
    w_down_scale: float = 1.0,
) -> Workload:
    """Draw one layer's inputs.

    x_kind: "normal" -> x ~ N(0,1); "rmsnorm" -> N(0,1) rows divided by
    sqrt(mean(row^2) + 1e-6) (no gain). Weights use std 1/sqrt(fan_in):
    d for W_up/W_gate, f for W_down0 (times w_down_scale). ids are uniform
    in [0, vocab).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    rng = np.random.default_rng(seed)
    W_up = _normal(rng, (f, d), 1.0 / np.sqrt(d))
    W_gate = _normal(rng, (f, d), 1.0 / np.sqrt(d))
    W_down0 = _normal(rng, (d, f), w_down_scale / np.sqrt(f))
    E_tgt = _normal(rng, (vocab, d), e_std)
    x = rng.standard_normal(size=(B, T, d), dtype=np.float32)
    if x_kind == "rmsnorm":
        ms = np.mean(x.astype(np.float64) ** 2, axis=-1, keepdims=True)
        x = (x / np.sqrt(ms + 1e-6)).astype(np.float32)
    elif x_kind != "normal":
        raise ValueError("x_kind must be 'normal' or 'rmsnorm'")
    ids = rng.integers(0, vocab, size=(B, T + 1), dtype=np.int32)
    if dtype == "bf16":
        W_up, W_gate, W_down0, E_tgt, x = (bf16_round(a) for a in (W_up, W_gate, W_down0, E_tgt, x))
    return Workload(name=name, d=d, f=f, B=B, T=T, C=C, eta=float(eta), dtype=dtype, vocab=vocab,
                    W_up=W_up, W_gate=W_gate, W_down0=W_down0, E_tgt=E_tgt, x=x, ids=ids,
                    meta={"seed": seed, "x_kind": x_kind, "e_std": e_std})


# The five workloads. c4 is the long-stream headline; it is swept over C in {128, 256}.
CONFIGS: Dict[str, Dict[str, object]] = {
    "c1_tiny_f32": dict(d=64, f=256, B=1, T=1024, C=128, eta=0.01, dtype="f32", vocab=512,
                        e_std=1.0, x_kind="normal", seed=1),
    "c2_1k4k_b4": dict(d=1024, f=4096, B=4, T=8192, C=256, eta=1e-3, dtype="bf16", vocab=32000,
                       e_std=0.02, x_kind="normal", seed=2),
    "c3_4b_32k": dict(d=2560, f=9728, B=1, T=32768, C=256, eta=1e-3, dtype="bf16", vocab=151936,
                      e_std=0.02, x_kind="rmsnorm", seed=3),
    "c4_4b_128k": dict(d=2560, f=9728, B=1, T=131072, C=256, eta=1e-3, dtype="bf16", vocab=151936,
                       e_std=0.02, x_kind="rmsnorm", seed=4),
    # per layer; the stack has 36 such layers, layer l seeded with (5, l)
    "c5_4b_stack36": dict(d=2560, f=9728, B=2, T=16384, C=256, eta=1e-3, dtype="bf16", vocab=151936,
                          e_std=0.02, x_kind="normal", seed=(5, 0)),
}

C5_LAYERS = 36


def make_config(name: str, *, T: Optional[int] = None, C: Optional[int] = None, B: Optional[int] = None,
                seed=None) -> Workload:
    """Inputs of a named workload; T, C, B and seed may be overridden (e.g. a
    shorter stream of the same layer shape, or c5's per-layer seed (5, l))."""
    cfg = dict(CONFIGS[name])
    if T is not None:
        cfg["T"] = T
    if C is not None:
        cfg["C"] = C
    if B is not None:
        cfg["B"] = B
    if seed is not None:
        cfg["seed"] = seed
    return make_inputs(name=name, **cfg)


def make_target_conv(d: int, K: int = 5, dtype: str = "bf16", seed=0) -> Tuple[np.ndarray, np.ndarray]:
    """Weights of the general target: conv_w [K][d] depthwise taps with std
    1/sqrt(K), and W_target [d][d] = I + N(0, 1/d) (a diagonal-dominant
    projection, as the pages start it from a diagonal form). Drawn in fp32 and,
    for bf16, rounded once (RNE)."""
    rng = np.random.default_rng(seed)
    cw = _normal(rng, (K, d), 1.0 / np.sqrt(K))
    Wt = np.eye(d, dtype=np.float32) + _normal(rng, (d, d), 1.0 / np.sqrt(d))
    if dtype == "bf16":
        cw, Wt = bf16_round(cw), bf16_round(Wt)
    return cw.astype(np.float32), Wt.astype(np.float32)


def shape_of(name: str) -> Tuple[int, int, int, int, int]:
    c = CONFIGS[name]
    return c["d"], c["f"], c["B"], c["T"], c["C"]
