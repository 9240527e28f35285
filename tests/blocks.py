"""Constructed MX blocks that reach every finite bf16 value at every useful block exponent.

Each block holds 31 test values and one "setter" 448 * 2^k, the largest magnitude allowed for a
block whose E8M0 exponent is k, so the block's exponent is exactly k for every test value x with
|x| <= 448 * 2^k. For each x, k runs from the smallest such exponent upward (twelve steps cover
every k at which x does not round to zero; beyond that every code is a zero).
"""
from __future__ import annotations

import numpy as np

import bruteforce as bf

K_STEPS = 12


def finite_bf16_bits() -> np.ndarray:
    u = np.arange(65536, dtype=np.uint32)
    return u[((u >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def exhaustive_blocks() -> tuple[np.ndarray, np.ndarray]:
    """(blocks [n, 32] of bf16 bits, k [n]) with n a multiple of 128."""
    xs = finite_bf16_bits()
    k0 = bf.e8m0_search(np.abs(bf.bf16_values(xs)))
    out_blocks, out_k = [], []
    for step in range(K_STEPS):
        k = k0 + step
        ok = k <= 119  # the setter 448 * 2^k must be a finite bf16
        for kk in np.unique(k[ok]):
            vals = xs[ok & (k == kk)]
            setter_bits = np.uint16((np.float32(448.0 * 2.0 ** kk)).view(np.uint32) >> 16)
            nb = -(-len(vals) // 31)
            pad = np.full(nb * 31 - len(vals), setter_bits, np.uint16)
            body = np.concatenate([vals, pad]).reshape(nb, 31)
            blk = np.concatenate([body, np.full((nb, 1), setter_bits, np.uint16)], axis=1)
            out_blocks.append(blk)
            out_k.append(np.full(nb, kk))
    blocks = np.concatenate(out_blocks)
    ks = np.concatenate(out_k)
    n = len(blocks)
    extra = (-n) % 128
    blocks = np.concatenate([blocks, np.zeros((extra, 32), np.uint16)])
    ks = np.concatenate([ks, np.full(extra, -127)])
    return blocks, ks


def expected_codes(blocks: np.ndarray, ks: np.ndarray) -> np.ndarray:
    vals = bf.bf16_values(blocks)
    return bf.encode_nearest(vals * np.ldexp(1.0, -ks)[:, None])


def as_rowwise_input(blocks: np.ndarray) -> np.ndarray:
    """[1, n/4, 1, 128]: four consecutive blocks per D=128 row."""
    return np.ascontiguousarray(blocks.reshape(1, -1, 1, 128))


def as_v_input(blocks: np.ndarray) -> np.ndarray:
    """[1, 32*(n/128), 1, 128]: block m sits in column d = m % 128, token block u = m // 128."""
    n = len(blocks)
    U = n // 128
    v = blocks.reshape(U, 128, 32).transpose(0, 2, 1).reshape(1, U * 32, 1, 128)
    return np.ascontiguousarray(v)
