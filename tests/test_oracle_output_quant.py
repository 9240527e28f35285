"""Pins of the oracle's MXFP8 encoding of real-valued rows (the block-scaled output, E4M3 codes with
one E8M0 per 32 elements of D): it agrees with the rowwise input quantiser on bf16 values, values on
the E4M3 grid of their block round-trip exactly, and the error of any value is within half an E4M3
step of its block."""
import numpy as np

import oracle
from causal_mxfp8_block_amd.inputs import bf16_bits, bf16_to_f32


def _decode(codes, scales):
    dec = np.vectorize(oracle.e4m3_decode)(codes.astype(np.int64))
    k = scales.astype(np.int64) - 127
    return dec * np.ldexp(1.0, np.repeat(k, 32, axis=-1))


def test_matches_rowwise_quantiser_on_bf16_rows():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 8, 3, 128)).astype(np.float32) * np.float32(2.0) ** rng.integers(-20, 20, (1, 8, 3, 1))
    bits = bf16_bits(x)
    c0, s0 = oracle.quantize_rowwise(oracle.BF16View.bshd(bits))           # [B,H,S,D]
    vals = bf16_to_f32(bits).astype(np.float64).transpose(0, 2, 1, 3)       # [B,H,S,D]
    c1, s1 = oracle.quantize_rows(vals)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


def test_grid_values_round_trip_exactly():
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, size=(64, 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    k = rng.integers(-30, 30, size=(64, 4))
    x = np.vectorize(oracle.e4m3_decode)(codes.astype(np.int64)) * np.ldexp(1.0, np.repeat(k, 32, axis=1))
    c, s = oracle.quantize_rows(x)
    assert np.array_equal(_decode(c, s), x)


def test_error_within_half_step():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((256, 128)) * np.exp(rng.uniform(-8, 8, size=(256, 1)))
    x[3, :32] = 0.0  # an all-zero block: byte 0, codes 0
    c, s = oracle.quantize_rows(x)
    assert s[3, 0] == 0 and np.all(c[3, :32] == 0)
    err = np.abs(_decode(c, s) - x)
    k = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    # normal E4M3 values: half a step is 2^-4 of the value; subnormals: 2^-10 of the block scale
    assert np.all(err <= np.maximum(np.ldexp(np.abs(x), -4), np.ldexp(1.0, k - 10)) * (1 + 1e-12))
    amax = np.abs(x).reshape(256, 4, 32).max(axis=2)
    # the scale is the smallest power of two that fits the block: amax <= 448 * 2^k < 896 * 2^k
    kk = s.astype(np.int64) - 127
    assert np.all(amax <= 448 * np.ldexp(1.0, kk)) and np.all((amax > 448 * np.ldexp(1.0, kk - 1)) | (amax == 0))
