"""Seeded synthetic inputs shaped like the benchmark workloads of TransformerEngine PR #3865
(section "Performance": batch 1, 16 query heads, 4 or 16 KV heads, D = 128, causal, BSHD).

This module holds none of the method's arithmetic: it draws random bf16 tensors and nothing else,
so both the product's tests/benchmark and the CPU oracle may use it.

Recipe (the pages name no dataset; random tensors of the benchmark's shapes stand in for it):
  * ``numpy.random.Generator(PCG64(seed))``; Q, K, V drawn in that order as
    ``standard_normal(float32)`` in logical [B,S,H,D] order; then the workload's extras;
  * extras: ``outliers`` multiplies 1% of V entries (``rng.random(V.shape) < 0.01``) by 64;
    ``token_amplitudes`` multiplies each (token, kv-head) row of V by 2**e, e ~ U{-4..4};
  * cast to bf16 with round-to-nearest-even (both extras are exact powers of two);
  * SBHD workloads are the same logical draw permuted to [S,B,H,D] and made contiguous.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    layout: str  # "bshd" or "sbhd"
    values: str  # "normal", "outliers", "token_amplitudes"
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.D)))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_s128", 1, 1, 1, 128, 128, "bshd", "normal", 0),
        Workload("gqa16x4_s8k_outliers", 1, 16, 4, 8192, 128, "bshd", "outliers", 1),
        Workload("mha16_s16k", 1, 16, 16, 16384, 128, "bshd", "normal", 2),
        Workload("gqa16x4_s32k_amplitudes", 1, 16, 4, 32768, 128, "bshd", "token_amplitudes", 3),
        Workload("mha16_s32k_sbhd", 1, 16, 16, 32768, 128, "sbhd", "normal", 4),
    ]
}
HEADLINE = "gqa16x4_s32k_amplitudes"


def custom(B, Hq, Hkv, S, D=128, layout="bshd", values="normal", seed=0, name="custom") -> Workload:
    return Workload(name, B, Hq, Hkv, S, D, layout, values, seed)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even. Inputs must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng: np.random.Generator, w: Workload, S: int):
    q = rng.standard_normal((w.B, S, w.Hq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, S, w.Hkv, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, S, w.Hkv, w.D), dtype=np.float32)
    if w.values == "outliers":
        mask = rng.random(v.shape) < 0.01
        v[mask] *= np.float32(64.0)
    elif w.values == "token_amplitudes":
        e = rng.integers(-4, 5, size=(w.B, S, w.Hkv))
        v *= np.ldexp(np.float32(1.0), e).astype(np.float32)[..., None]
    elif w.values != "normal":
        raise ValueError(w.values)
    return q, k, v


@dataclass
class Inputs:
    """bf16 bit patterns in the workload's storage layout ([B,S,H,D] or [S,B,H,D])."""
    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    def logical(self, name: str) -> np.ndarray:
        """[B,S,H,D] view of q, k or v."""
        x = getattr(self, name)
        return x if self.workload.layout == "bshd" else x.transpose(1, 0, 2, 3)


def _store(w: Workload, x: np.ndarray) -> np.ndarray:
    b = bf16_bits(x)
    if w.layout == "sbhd":
        b = np.ascontiguousarray(b.transpose(1, 0, 2, 3))
    return b


def make_inputs(w: Workload | str, seed: int | None = None) -> Inputs:
    if isinstance(w, str):
        w = WORKLOADS[w]
    if seed is not None:
        w = replace(w, seed=seed)
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q, k, v = _draw(rng, w, w.S)
    return Inputs(w, _store(w, q), _store(w, k), _store(w, v))


def perturb_after(inp: Inputs, t: int, outlier_at_next: bool = False) -> Inputs:
    """Copy of ``inp`` whose tokens > t are re-drawn (same distribution) from PCG64((seed, t)).

    With ``outlier_at_next`` the V row of token t+1 is also multiplied by 64 (exact in bf16): the
    planted outlier that raises a shared columnwise V scale of t's own 32-token block.
    """
    w = inp.workload
    n = w.S - (t + 1)
    q, k, v = (inp.logical(x).copy() for x in ("q", "k", "v"))
    if n > 0:
        rng = np.random.Generator(np.random.PCG64([w.seed, t]))
        dq, dk, dv = _draw(rng, w, n)
        q[:, t + 1:] = bf16_bits(dq)
        k[:, t + 1:] = bf16_bits(dk)
        v[:, t + 1:] = bf16_bits(dv)
        if outlier_at_next:
            v[:, t + 1] = bf16_bits(bf16_to_f32(v[:, t + 1]) * np.float32(64.0))
    relayout = (lambda a: a) if w.layout == "bshd" else (lambda a: np.ascontiguousarray(a.transpose(1, 0, 2, 3)))
    return Inputs(w, relayout(q), relayout(k), relayout(v))
