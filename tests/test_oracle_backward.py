"""Pins of the oracle's backward on decoded operands (causal softmax attention gradients with the
forward's O and lse as statistics): a finite-difference gradient check of the scalar sum(dO * O)
against a textbook causal attention forward, the GQA identity (shared KV heads = the sum over the
group with repeated KV), row subsets, and the code-level entry point = the value-level one on the
decoded operands."""
import numpy as np
import pytest

import oracle
from causal_mxfp8_block_amd.inputs import bf16_bits, bf16_to_f32


def _forward(Q, K, V, scale):
    """Textbook causal attention in fp64: O [B,Hq,S,D], lse [B,Hq,S] (K, V repeated over groups)."""
    G = Q.shape[1] // K.shape[1]
    Kr, Vr = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    s = scale * np.einsum("bhid,bhjd->bhij", Q, Kr)
    S = Q.shape[2]
    s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=-1, keepdims=True)
    return np.einsum("bhij,bhjd->bhid", p / l, Vr), (m + np.log(l))[..., 0]


def _rand(shape, rng):
    return rng.standard_normal(shape)


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(40)
    B, Hq, Hkv, S, D, scale = 1, 2, 1, 40, 128, 0.0884
    Q, K, V = _rand((B, Hq, S, D), rng), _rand((B, Hkv, S, D), rng), _rand((B, Hkv, S, D), rng)
    dO = _rand((B, Hq, S, D), rng)
    O, lse = _forward(Q, K, V, scale)
    dq, dk, dv = oracle.attn_bwd_values(Q, K, V, O, dO, lse, scale)
    f = lambda q, k, v: float(np.sum(dO * _forward(q, k, v, scale)[0]))
    eps = 1e-6
    for name, X, G in (("Q", Q, dq), ("K", K, dk), ("V", V, dv)):
        for _ in range(25):
            idx = tuple(int(rng.integers(0, n)) for n in X.shape)
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = dict(Q=Q, K=K, V=V)
            args_m = dict(Q=Q, K=K, V=V)
            args_p[name], args_m[name] = Xp, Xm
            fd = (f(args_p["Q"], args_p["K"], args_p["V"]) - f(args_m["Q"], args_m["K"], args_m["V"])) / (2 * eps)
            assert abs(fd - G[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, G[idx])


def test_gqa_is_the_sum_over_the_group():
    rng = np.random.default_rng(41)
    B, Hq, Hkv, S, D, scale = 2, 4, 2, 70, 128, 0.0884
    Q, K, V = _rand((B, Hq, S, D), rng), _rand((B, Hkv, S, D), rng), _rand((B, Hkv, S, D), rng)
    dO = _rand((B, Hq, S, D), rng)
    O, lse = _forward(Q, K, V, scale)
    dq, dk, dv = oracle.attn_bwd_values(Q, K, V, O, dO, lse, scale)
    G = Hq // Hkv
    dq2, dk2, dv2 = oracle.attn_bwd_values(Q, np.repeat(K, G, axis=1), np.repeat(V, G, axis=1), O, dO, lse, scale)
    assert np.allclose(dq, dq2, rtol=1e-12, atol=1e-12)
    assert np.allclose(dk, dk2.reshape(B, Hkv, G, S, D).sum(axis=2), rtol=1e-12, atol=1e-12)
    assert np.allclose(dv, dv2.reshape(B, Hkv, G, S, D).sum(axis=2), rtol=1e-12, atol=1e-12)


def test_row_subsets():
    rng = np.random.default_rng(42)
    B, Hq, Hkv, S, D, scale = 1, 2, 2, 96, 128, 0.0884
    Q, K, V = _rand((B, Hq, S, D), rng), _rand((B, Hkv, S, D), rng), _rand((B, Hkv, S, D), rng)
    dO = _rand((B, Hq, S, D), rng)
    O, lse = _forward(Q, K, V, scale)
    dq, dk, dv = oracle.attn_bwd_values(Q, K, V, O, dO, lse, scale)
    rows = np.array([0, 5, 31, 32, 95], np.int32)
    dqs, dks, dvs = oracle.attn_bwd_values(Q, K, V, O, dO, lse, scale, qrows=rows, krows=rows)
    assert np.array_equal(dqs, dq[:, :, rows]) and np.array_equal(dks, dk[:, :, rows])
    assert np.array_equal(dvs, dv[:, :, rows])


def test_codes_entry_equals_values_entry_on_decoded_operands():
    rng = np.random.default_rng(43)
    B, Hq, Hkv, S, D, scale = 1, 2, 1, 64, 128, 0.0884
    q = bf16_bits(rng.standard_normal((B, S, Hq, D)).astype(np.float32))
    k = bf16_bits(rng.standard_normal((B, S, Hkv, D)).astype(np.float32))
    v = bf16_bits((rng.standard_normal((B, S, Hkv, D)) * 2.0 ** rng.integers(-4, 5, (B, S, Hkv, 1))).astype(np.float32))
    z = oracle.quantize_all(oracle.BF16View.bshd(q), oracle.BF16View.bshd(k), oracle.BF16View.bshd(v))
    dec = np.vectorize(oracle.e4m3_decode)
    Qd = dec(z.qc.astype(np.int64)) * np.ldexp(1.0, np.repeat(z.qs.astype(np.int64) - 127, 32, axis=-1))
    Kd = dec(z.kc.astype(np.int64)) * np.ldexp(1.0, np.repeat(z.ks.astype(np.int64) - 127, 32, axis=-1))
    Vd = dec(z.vt.astype(np.int64)) * np.ldexp(1.0, z.vta.astype(np.int64) - 127)[..., None]
    o = bf16_bits(rng.standard_normal((B, S, Hq, D)).astype(np.float32) * np.float32(0.3))
    do = bf16_bits(rng.standard_normal((B, S, Hq, D)).astype(np.float32))
    lse = (rng.standard_normal((B, Hq, S)) + 3.0).astype(np.float32)
    g = oracle.attn_bwd(z.qc, z.qs, z.kc, z.ks, z.vt, z.vta, oracle.BF16View.bshd(o), lse, oracle.BF16View.bshd(do),
                        scale)
    to = lambda x: bf16_to_f32(x).astype(np.float64).transpose(0, 2, 1, 3)
    h = oracle.attn_bwd_values(Qd, Kd, Vd, to(o), to(do), lse.astype(np.float64), float(np.float32(scale)))
    for a, b in zip(g, h):
        assert np.array_equal(a, b)


def test_bf16_rounding_allowance_covers_rounded_operands():
    """R16 pin: gradients computed with P and dS rounded to bf16 before their products (a model of
    the bf16 kernel) differ from the exact ones by at most the allowance, and the allowance is
    exercised (the rounding moves the gradients)."""
    rng = np.random.default_rng(44)
    B, Hq, Hkv, S, D, scale = 1, 2, 1, 96, 128, 0.0884
    Q, K, V = _rand((B, Hq, S, D), rng), _rand((B, Hkv, S, D), rng), _rand((B, Hkv, S, D), rng) * 4
    dO = _rand((B, Hq, S, D), rng)
    O, lse = _forward(Q, K, V, scale)
    O = O + 0.01 * _rand(O.shape, rng)  # statistics need not be those of Q, K, V exactly
    dq, dk, dv, aq, ak, av = oracle.attn_bwd_values(Q, K, V, O, dO, lse, scale, allowance=True)
    G = Hq // Hkv
    Kr, Vr = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    p = np.exp(scale * np.einsum("bhid,bhjd->bhij", Q, Kr) - lse[..., None])
    p = np.where(np.tril(np.ones((S, S), bool)), p, 0.0)
    delta = np.sum(dO * O, axis=-1)
    ds = p * (np.einsum("bhid,bhjd->bhij", dO, Vr) - delta[..., None])
    rb = lambda x: bf16_to_f32(bf16_bits(x.astype(np.float32))).astype(np.float64)
    pb, dsb = rb(p), rb(ds)
    mq = scale * np.einsum("bhij,bhjd->bhid", dsb, Kr)
    mk = scale * np.einsum("bhij,bhid->bhjd", dsb, Q).reshape(B, Hkv, G, S, D).sum(axis=2)
    mv = np.einsum("bhij,bhid->bhjd", pb, dO).reshape(B, Hkv, G, S, D).sum(axis=2)
    for m, ref, al in ((mq, dq, aq), (mk, dk, ak), (mv, dv, av)):
        assert np.all(np.abs(m - ref) <= al * (1 + 1e-9) + 1e-12)
        assert np.max(np.abs(m - ref)) > 0
