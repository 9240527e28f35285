"""GPU backward on decoded operands (attn_bwd) against the oracle, and its causality on the GPU.

The oracle gets no input from the GPU: O and lse come from the oracle's own leak-free forward
(rounded to bf16 and fp32, the types the backward takes), and the same O, lse and dO feed both sides.
Tolerance: P and dS enter the bf16 MFMAs rounded to bf16 (reading R16: the oracle bounds the effect
of that rounding per element, its allowance) and the outputs are bf16 (rounding error at most 2^-8
of the value), with fp32 accumulation: max(|err| - allowance - 2^-8 |ref|) <= 2e-2 RMS(ref)."""
import numpy as np
import pytest
import torch

import oracle
import causal_mxfp8_block_amd as mx
from causal_mxfp8_block_amd.inputs import bf16_bits, bf16_to_f32, custom, make_inputs, perturb_after
from gpu_helpers import gpu_quantize, oracle_view, say, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-2
REL = 2.0 ** -8


def _dout(inp, seed):
    w = inp.workload
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((w.B, w.S, w.Hq, w.D)).astype(np.float32)
    return bf16_bits(g) if w.layout == "bshd" else np.ascontiguousarray(bf16_bits(g).transpose(1, 0, 2, 3))


def _stats_from_oracle(inp, z):
    """O (bf16 bits in the inputs' layout) and lse (fp32 [B,Hq,S]) of the oracle's forward."""
    w = inp.workload
    o, lse, _ = oracle.forward(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"), w.scale, quant=z)
    ob = bf16_bits(o.astype(np.float32).transpose(0, 2, 1, 3))  # [B,S,Hq,D]
    if w.layout == "sbhd":
        ob = np.ascontiguousarray(ob.transpose(1, 0, 2, 3))
    return ob, lse.astype(np.float32)


def _view(bits, layout):
    return oracle.BF16View.sbhd(bits) if layout == "sbhd" else oracle.BF16View.bshd(bits)


def _gpu_bwd(inp, obits, lse, gbits):
    w = inp.workload
    g = gpu_quantize(inp)
    dq, dk, dv = mx.attn_bwd(g["qc"], g["qs"], g["kc"], g["ks"], g["vt"], g["vta"], to_dev(obits),
                             torch.from_numpy(lse).cuda(), to_dev(gbits), w.scale, layout=w.layout)
    torch.cuda.synchronize()
    to = (lambda t: t.permute(0, 2, 1, 3)) if w.layout == "bshd" else (lambda t: t.permute(1, 2, 0, 3))
    return [to(t).float().double().cpu().numpy() for t in (dq, dk, dv)]


def _gate(name, got, ref, al):
    rms = np.sqrt(np.mean(ref ** 2))
    excess = np.abs(got - ref) - al - REL * np.abs(ref)
    ratio = excess.max() / rms
    say(f"[{name}] max|err|/rms = {np.abs(got - ref).max() / rms:.3e}  max(|err| - allow - 2^-8|ref|)/rms = "
        f"{ratio:.3e}  mean(allow)/rms = {al.mean() / rms:.2e}  rms = {rms:.3e}")
    return ratio


# (1, 2, 2, 32): one block, so each kernel's loop runs a single step; (1, 8, 1, 96): eight query
# heads per KV head in the dK/dV sum
@pytest.mark.parametrize("shape", [(1, 1, 1, 128), (2, 4, 2, 288), (1, 2, 1, 96), (1, 3, 3, 64), (1, 4, 1, 416),
                                   (1, 2, 2, 32), (1, 8, 1, 96)])
def test_backward_matches_oracle_small(shape):
    B, Hq, Hkv, S = shape
    inp = make_inputs(custom(B, Hq, Hkv, S, values="token_amplitudes", seed=50 + sum(shape)))
    w = inp.workload
    say(f"backward {shape}")
    z = oracle.quantize_all(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"))
    obits, lse = _stats_from_oracle(inp, z)
    gbits = _dout(inp, 60 + sum(shape))
    dq, dk, dv = _gpu_bwd(inp, obits, lse, gbits)
    rq, rk, rv, aq, ak, av = oracle.attn_bwd(z.qc, z.qs, z.kc, z.ks, z.vt, z.vta, _view(obits, w.layout), lse,
                                             _view(gbits, w.layout), w.scale, allowance=True)
    for name, got, ref, al in (("dq", dq, rq, aq), ("dk", dk, rk, ak), ("dv", dv, rv, av)):
        assert _gate(f"{name} {shape}", got, ref, al) <= TOL


def test_backward_matches_oracle_s32k_two_heads():
    """The SBHD S=32K MHA workload (the forward-plus-backward configuration), two of its heads (heads
    are independent; the launch geometry per head is that of the full run), on sampled query rows
    (dQ) and key rows (dK, dV)."""
    full = make_inputs("mha16_s32k_sbhd")
    w = full.workload
    from causal_mxfp8_block_amd.inputs import Inputs, Workload
    import dataclasses
    w2 = dataclasses.replace(w, Hq=2, Hkv=2, name=w.name + "_2heads")
    inp = Inputs(w2, np.ascontiguousarray(full.q[:, :, :2]), np.ascontiguousarray(full.k[:, :, :2]),
                 np.ascontiguousarray(full.v[:, :, :2]))
    say("backward s32k two heads")
    z = oracle.quantize_all(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"))
    obits, lse = _stats_from_oracle(inp, z)
    gbits = _dout(inp, 5)
    dq, dk, dv = _gpu_bwd(inp, obits, lse, gbits)
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([np.arange(64), rng.integers(0, w2.S, 96), np.arange(w2.S - 32, w2.S)]))
    rows = rows.astype(np.int32)
    rq, rk, rv, aq, ak, av = oracle.attn_bwd(z.qc, z.qs, z.kc, z.ks, z.vt, z.vta, _view(obits, "sbhd"), lse,
                                             _view(gbits, "sbhd"), w2.scale, qrows=rows, krows=rows, allowance=True)
    for name, got, ref, al in (("dq", dq[:, :, rows], rq, aq), ("dk", dk[:, :, rows], rk, ak),
                               ("dv", dv[:, :, rows], rv, av)):
        assert _gate(f"{name} s32k", got, ref, al) <= TOL


def test_backward_gqa_is_the_group_sum():
    """dK, dV with shared KV heads = the sums over the group of the run with the KV heads repeated."""
    inp = make_inputs(custom(1, 4, 2, 160, values="normal", seed=71))
    w = inp.workload
    z = oracle.quantize_all(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"))
    obits, lse = _stats_from_oracle(inp, z)
    gbits = _dout(inp, 72)
    dq, dk, dv = _gpu_bwd(inp, obits, lse, gbits)
    from causal_mxfp8_block_amd.inputs import Inputs
    import dataclasses
    rep = Inputs(dataclasses.replace(w, Hkv=4), inp.q, np.repeat(inp.k, 2, axis=2), np.repeat(inp.v, 2, axis=2))
    dq2, dk2, dv2 = _gpu_bwd(rep, obits, lse, gbits)
    assert np.array_equal(dq, dq2)
    for got, full in ((dk, dk2), (dv, dv2)):
        s = full.reshape(1, 2, 2, 160, 128).sum(axis=2)
        # one bf16 rounding (2^-8 relative) of the sum against one of each part: 2^-8 (|a| + |b| + |a + b|)
        # <= 2^-7 (|a| + |b|)
        assert np.all(np.abs(got - s) <= 2.0 ** -7 * (np.abs(full).reshape(1, 2, 2, 160, 128).sum(axis=2)) + 1e-30)


def test_backward_dq_is_causal_on_gpu():
    """Tokens > t (Q, K, V and dO) re-drawn, with a x64 V outlier at t+1: the leak-free forward's rows
    <= t and the backward's dQ rows <= t are bit-identical (the decoded operands of a token depend on
    that token only)."""
    inp = make_inputs("tiny_s128")
    w = inp.workload

    def run(x, gbits):
        q, k, v = (to_dev(getattr(x, n)) for n in ("q", "k", "v"))
        o, lse = mx.attn_fwd(q, k, v, w.scale, layout=w.layout)
        g = gpu_quantize(x)
        dq, _, _ = mx.attn_bwd(g["qc"], g["qs"], g["kc"], g["ks"], g["vt"], g["vta"], o, lse, to_dev(gbits), w.scale,
                               layout=w.layout)
        torch.cuda.synchronize()
        return dq.cpu()

    g0 = _dout(inp, 81)
    base = run(inp, g0)
    for t in (0, 5, 31, 32, 40, 63, 100, 126):
        pert = perturb_after(inp, t, outlier_at_next=True)
        g1 = g0.copy()
        g1[:, t + 1:] = _dout(pert, 82 + t)[:, t + 1:]
        dq = run(pert, g1)
        assert torch.equal(dq[:, :t + 1], base[:, :t + 1]), t
