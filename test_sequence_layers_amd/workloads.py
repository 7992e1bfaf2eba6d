"""Seeded synthetic workloads for the TTT-layer forward pass.

This module only draws and formats inputs: it holds none of the method's arithmetic, and
both the GPU tests/benchmark and the CPU oracle consume exactly the arrays it returns.

Recipe (every workload): numpy PCG64 generator seeded with the given seed; draw Q, K, V as
float32 standard normal of shape [B, H, T, d] in that order, then the initial state
(W0 [H, d, d], or W1 [H, h, d] then W2 [H, d, h]) as N(0, 0.02^2) float32 unless the
workload starts from zero.  Where the workload asks for unit keys, each k_t is divided by
its float32 L2 norm.  For bf16 workloads Q, K, V are then rounded to bfloat16 with
round-to-nearest-even, so the float32 arrays returned here hold exactly the bf16 values the
GPU reads.  States are always float32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "round_to_bf16"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str           # "linear", "delta" (b = 1 delta rule) or "mlp"
    B: int
    H: int
    T: int
    d: int
    chunk: int
    causal: bool
    eta: float
    io: str             # "f32" or "bf16"
    unit_keys: bool
    init: str           # "zero" or "normal" (N(0, 0.02^2))
    h: int = 0          # MLP hidden width
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T


# The five workloads the method is measured on.  Index i uses seed 1000 + i.
WORKLOADS = [
    # TTT-Linear, tiny fp32 case.
    Workload("linear_tiny_fp32", "linear", B=1, H=1, T=64, d=16, chunk=16, causal=True,
             eta=0.1, io="f32", unit_keys=True, init="zero", seed=1000),
    # TTT-Linear at d = 64, T = 2048 (the headline throughput case).
    # eta = (1.0 / d) * 8 read left to right = 0.125.
    Workload("linear_d64_T2048", "linear", B=8, H=12, T=2048, d=64, chunk=16, causal=True,
             eta=0.125, io="bf16", unit_keys=True, init="normal", seed=1001),
    # Exact delta rule (mini-batch of one token), long sequences.
    Workload("delta_d64_T8192", "delta", B=4, H=16, T=8192, d=64, chunk=1, causal=True,
             eta=0.5, io="bf16", unit_keys=True, init="zero", seed=1002),
    # TTT-MLP, hidden 4 d, d = 64, T = 2048.  Keys are unit-normalised here although the
    # workload statement leaves them raw: with raw N(0, 1) keys (|k|^2 ~ 64), eta = 0.1 and
    # 16 summed gradients the recurrence itself overflows to inf/NaN within 256 tokens in
    # float64, so there is nothing finite to reproduce.  Unit keys keep it finite.
    Workload("mlp_h256_T2048", "mlp", B=8, H=12, T=2048, d=64, h=256, chunk=16, causal=True,
             eta=0.1, io="bf16", unit_keys=True, init="normal", seed=1003),
    # Non-causal full-batch MLP (one chunk of all 196 tokens of a 14 x 14 grid), hidden = d.
    Workload("mlp_vision_N196", "mlp", B=64, H=6, T=196, d=64, h=64, chunk=196, causal=False,
             eta=1.0, io="bf16", unit_keys=False, init="normal", seed=1004),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32)
    # NaN stays NaN (never produced by the generators, kept for completeness).
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC00000
    return out.view(np.float32)


def make_inputs(w: Workload, seed: Optional[int] = None, **overrides) -> dict:
    """Draw the inputs of workload `w` (any field may be overridden, e.g. B=1, T=100).

    Returns a dict with float32 arrays q, k, v [B, H, T, d] and either w0 [H, d, d]
    (linear / delta) or w1 [H, h, d] and w2 [H, d, h] (mlp), plus the Workload used.
    """
    if overrides:
        w = w.replace(**overrides)
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.T, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    out = {"workload": w}
    if w.kind in ("linear", "delta"):
        if w.init == "zero":
            out["w0"] = np.zeros((w.H, w.d, w.d), np.float32)
        else:
            out["w0"] = (0.02 * rng.standard_normal((w.H, w.d, w.d), dtype=np.float32))
    else:
        if w.init == "zero":
            out["w1"] = np.zeros((w.H, w.h, w.d), np.float32)
            out["w2"] = np.zeros((w.H, w.d, w.h), np.float32)
        else:
            out["w1"] = (0.02 * rng.standard_normal((w.H, w.h, w.d), dtype=np.float32))
            out["w2"] = (0.02 * rng.standard_normal((w.H, w.d, w.h), dtype=np.float32))
    if w.unit_keys:
        n = np.sqrt(np.sum(k * k, axis=-1, keepdims=True, dtype=np.float32))
        k = (k / n).astype(np.float32)
    if w.io == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    out["q"], out["k"], out["v"] = q, k, v
    return out


def make_token_rates(w: Workload, seed: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Seeded per-token rate factors [B, H, T] float32, uniform in [lo, hi): the range of a
    sigmoid gate.  A separate stream, so the workload's other inputs are unchanged."""
    rng = np.random.default_rng(10_000 + seed)
    return rng.uniform(lo, hi, size=(w.B, w.H, w.T)).astype(np.float32)


def make_ln_params(w: Workload, seed: int) -> tuple:
    """Seeded per-head layer-norm gain and bias, float32 [H, d] each: gain 1 + 0.1 N(0, 1),
    bias 0.1 N(0, 1) (near their usual initial values 1 and 0).  A separate stream."""
    rng = np.random.default_rng(20_000 + seed)
    gain = (1.0 + 0.1 * rng.standard_normal((w.H, w.d))).astype(np.float32)
    bias = (0.1 * rng.standard_normal((w.H, w.d))).astype(np.float32)
    return gain, bias
