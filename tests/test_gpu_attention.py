"""GPU parity of the attention kernels (completed-block partial, own-block partial, LSE merge and the
whole forward) against the oracle, plus the causality invariant, determinism, poisoned outputs,
layout and GQA identities on the HIP path.

Tolerance: attention outputs max|err| <= 2e-2 * RMS(oracle output) (fp32 output mode); the RMS is
that of the whole tensor, estimated from a seeded uniform sample of rows at full size. The kernel
forms its scores and P.V on the block-scaled FP8 MFMA, whose sums are not exact (reading R15): where
a P value of the completed blocks lies within the hardware error bound of a rounding boundary both
codes are valid results, and an element may in addition differ by the oracle's allowance. The gate
(gpu_helpers.gate) keeps that allowance's terms apart: every element over the plain tolerance must
have an alternative valid code in its row, the excess must fit the allowance, and at most 2e-3 of
the elements may exceed the plain tolerance. The own-block partial and the merge carry no
quantisation, only fp32 rounding: 1e-4 * RMS there."""
import numpy as np
import pytest
import torch

import oracle
import causal_mxfp8_block_amd as mx
from causal_mxfp8_block_amd.inputs import WORKLOADS, custom, make_inputs, perturb_after
from gpu_helpers import (gate, gpu_forward, gpu_quantize, oracle_view, report, sample_rows, say, to_dev,
                         uniform_rows)

pytestmark = pytest.mark.gpu
TOL = 2e-2
MAX_OVER = 2e-3  # largest fraction of elements allowed over the plain tolerance (code flips)


def _oracle_quant(inp):
    return oracle.quantize_all(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"))


def _partials_case(inp, rows=None):
    w = inp.workload
    g = gpu_quantize(inp)
    z = _oracle_quant(inp)
    for key in ("qc", "qs", "kc", "ks", "vc", "vcs", "vt", "vta"):
        assert np.array_equal(g[key].cpu().numpy(), getattr(z, key)), key
    oc, lc = mx.attn_fwd_completed_blocks(g["qc"], g["qs"], g["kc"], g["ks"], g["vc"], g["vcs"], w.scale)
    oo, lo = mx.attn_fwd_own_block(g["qc"], g["qs"], g["kc"], g["ks"], g["vt"], g["vta"], w.scale)
    torch.cuda.synchronize()
    roc, rlc, ral = oracle.attn_completed(z.qc, z.qs, z.kc, z.ks, z.vc, z.vcs, w.Hq, w.Hkv, w.scale, rows,
                                          allowance=True)
    roo, rlo = oracle.attn_own(z.qc, z.qs, z.kc, z.ks, z.vt, z.vta, w.Hq, w.Hkv, w.scale, rows)
    sel = slice(None) if rows is None else rows
    goc = oc.double().cpu().numpy()[:, :, sel]
    glc = lc.double().cpu().numpy()[:, :, sel]
    goo = oo.double().cpu().numpy()[:, :, sel]
    glo = lo.double().cpu().numpy()[:, :, sel]
    return (goc, glc, goo, glo), (roc, rlc, roo, rlo, ral)


@pytest.mark.parametrize("shape", [(1, 1, 1, 128), (2, 4, 2, 416), (1, 8, 2, 288), (1, 2, 1, 32), (1, 3, 1, 96),
                                   (1, 4, 2, 352)])
def test_partials_small(shape):
    """Both partials on shapes spanning several 128-query tiles, ragged tails (S % 128 != 0), GQA and
    batch, and odd numbers of 64-key tiles per workgroup (S = 352: five for the third query tile),
    compared with the oracle on every row."""
    B, Hq, Hkv, S = shape
    inp = make_inputs(custom(B, Hq, Hkv, S, values="outliers", seed=sum(shape)))
    say(f"partials {shape}")
    (goc, glc, goo, glo), (roc, rlc, roo, rlo, ral) = _partials_case(inp)
    n0 = min(32, S)
    assert np.all(goc[:, :, :n0] == 0) and np.all(np.isneginf(glc[:, :, :n0]))
    if S > 32:
        rms = np.sqrt(np.mean(roc[:, :, 32:] ** 2))
        gate("o_c", goc[:, :, 32:], roc[:, :, 32:], rms, allowance=ral.total[:, :, 32:],
             allowance_hw=ral.code[:, :, 32:] + ral.pv[:, :, 32:], tol=TOL, max_over_frac=MAX_OVER)
        assert np.max(np.abs(glc[:, :, 32:] - rlc[:, :, 32:])) < 1e-4
    rms_o = np.sqrt(np.mean(roo ** 2))
    assert report("o_o", goo, roo, rms_o) <= 1e-4
    assert np.max(np.abs(glo - rlo)) < 1e-4


def test_lse_merge_matches_oracle():
    rng = np.random.default_rng(4)
    B, H, S, D = 2, 3, 64, 128
    oc, oo = rng.standard_normal((2, B, H, S, D))
    lc, lo = rng.standard_normal((2, B, H, S)) * 4
    lc[:, :, :32] = -np.inf
    t = lambda a: torch.tensor(a, dtype=torch.float32, device="cuda:0")
    o32, l32 = mx.lse_merge(t(oc), t(lc), t(oo), t(lo), out_dtype=torch.float32)
    o16, l16 = mx.lse_merge(t(oc), t(lc), t(oo), t(lo), out_dtype=torch.bfloat16)
    osb, lsb = mx.lse_merge(t(oc), t(lc), t(oo), t(lo), out_dtype=torch.float32, layout="sbhd")
    torch.cuda.synchronize()
    f32 = lambda a: np.asarray(a, np.float32).astype(np.float64)
    ro, rl = oracle.lse_merge(f32(oc), f32(lc), f32(oo), f32(lo))
    go = o32.double().cpu().numpy().transpose(0, 2, 1, 3)
    assert report("merge", go, ro, np.sqrt(np.mean(ro ** 2))) <= 1e-5
    assert np.max(np.abs(l32.double().cpu().numpy() - rl)) < 1e-5
    # bf16 output is the round-to-nearest-even of the fp32 output
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(osb.permute(1, 0, 2, 3), o32) and torch.equal(lsb, l32)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_forward_parity_workloads(name):
    """The whole forward at every benchmark workload, in the launch configuration the benchmark times:
    sampled rows (all heads) vs the oracle, max|err| <= 2e-2 * RMS(O)."""
    inp = make_inputs(name)
    w = inp.workload
    say(f"forward parity {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} S={w.S} {w.layout} {w.values}")
    go, gl = gpu_forward(inp, torch.float32)
    if w.S <= 1024:
        rows, rms_rows = None, None
    else:
        rows, rms_rows = sample_rows(w.S, w.seed), uniform_rows(w.S, w.seed)
    z = _oracle_quant(inp)
    ro, rl, parts = oracle.forward(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"), w.scale,
                                   rows, quant=z)
    if rms_rows is None:
        rms = np.sqrt(np.mean(ro ** 2))
    else:
        ru, _, _ = oracle.forward(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"), w.scale,
                                  rms_rows, quant=z)
        rms = np.sqrt(np.mean(ru ** 2))
    sel = slice(None) if rows is None else rows
    gate(f"forward {name}", go[:, :, sel], ro, rms, rows, allowance=parts["allowance"],
         allowance_hw=parts["allowance_code"] + parts["allowance_pv"], tol=TOL, max_over_frac=MAX_OVER)
    assert np.max(np.abs(gl[:, :, sel] - rl)) < 1e-3


def test_completed_partial_full_size():
    """The completed-block kernel alone (attn_fwd_completed_blocks) at the benchmark workload's full
    size, on sampled rows of every head, against the oracle's completed partial."""
    inp = make_inputs("gqa16x4_s32k_amplitudes")
    w = inp.workload
    say(f"completed partial at full size: {w.name}")
    g = gpu_quantize(inp)
    oc, lc = mx.attn_fwd_completed_blocks(g["qc"], g["qs"], g["kc"], g["ks"], g["vc"], g["vcs"], w.scale)
    torch.cuda.synchronize()
    z = _oracle_quant(inp)
    rows = sample_rows(w.S, w.seed)
    rows = rows[rows >= 32]
    roc, rlc, ral = oracle.attn_completed(z.qc, z.qs, z.kc, z.ks, z.vc, z.vcs, w.Hq, w.Hkv, w.scale, rows,
                                          allowance=True)
    ru, _ = oracle.attn_completed(z.qc, z.qs, z.kc, z.ks, z.vc, z.vcs, w.Hq, w.Hkv, w.scale,
                                  uniform_rows(w.S, w.seed)[uniform_rows(w.S, w.seed) >= 32])
    rms = np.sqrt(np.mean(ru ** 2))
    goc = oc.double().cpu().numpy()[:, :, rows]
    glc = lc.double().cpu().numpy()[:, :, rows]
    gate("completed full size", goc, roc, rms, rows, allowance=ral.total, allowance_hw=ral.code + ral.pv, tol=TOL,
         max_over_frac=MAX_OVER)
    assert np.max(np.abs(glc - rlc)) < 1e-3


def test_bf16_output_is_rne_of_f32_output():
    inp = make_inputs(custom(1, 4, 2, 256, seed=8))
    q, k, v = (to_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    o32, l32 = mx.attn_fwd(q, k, v, out_dtype=torch.float32)
    o16, l16 = mx.attn_fwd(q, k, v, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(l16, l32)


def test_fused_entry_equals_attn_fwd_and_stepwise_path_matches_oracle():
    """attn_fwd (K, V quantised, Q inside the attention kernel) = quantise + attn_fwd_fused, bit for
    bit; the stepwise path (two partials and the
    merge as separate kernels) and the fused one both meet the oracle."""
    inp = make_inputs(custom(2, 4, 1, 224, values="token_amplitudes", seed=12))
    w = inp.workload
    q, k, v = (to_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    out, lse = mx.attn_fwd(q, k, v, out_dtype=torch.float32)
    g = gpu_quantize(inp)
    of, lf = mx.attn_fwd_fused(g["qc"], g["qs"], g["kc"], g["ks"], g["vc"], g["vcs"], g["vt"], g["vta"],
                               out_dtype=torch.float32)
    oc, lc = mx.attn_fwd_completed_blocks(g["qc"], g["qs"], g["kc"], g["ks"], g["vc"], g["vcs"])
    oo, lo = mx.attn_fwd_own_block(g["qc"], g["qs"], g["kc"], g["ks"], g["vt"], g["vta"])
    o2, l2 = mx.lse_merge(oc, lc, oo, lo, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out, of) and torch.equal(lse, lf)
    ro, rl, parts = oracle.forward(inp.q, inp.k, inp.v, w.scale)
    rms = np.sqrt(np.mean(ro ** 2))
    for name, o_, l_ in (("fused", of, lf), ("stepwise", o2, l2)):
        go = o_.double().cpu().numpy().transpose(0, 2, 1, 3)
        gate(name, go, ro, rms, allowance=parts["allowance"],
             allowance_hw=parts["allowance_code"] + parts["allowance_pv"], tol=TOL, max_over_frac=MAX_OVER)
        assert np.max(np.abs(l_.double().cpu().numpy() - rl)) < 1e-3


@pytest.mark.parametrize("shape,layout,values", [((1, 1, 1, 128), "bshd", "outliers"),
                                                  ((2, 4, 2, 416), "sbhd", "token_amplitudes"),
                                                  ((1, 8, 2, 288), "bshd", "normal"),
                                                  ((1, 3, 1, 96), "sbhd", "outliers")])
def test_bf16q_entry_equals_quantise_then_fused(shape, layout, values):
    """attn_fwd_fused_bf16q quantises Q inside the attention kernel: its output and LSE equal
    mxfp8_quantize(q) followed by attn_fwd_fused bit for bit, in both output dtypes, also when Q is a
    strided view (every other head of a wider tensor)."""
    B, Hq, Hkv, S = shape
    inp = make_inputs(custom(B, Hq, Hkv, S, layout=layout, values=values, seed=31 + S))
    g = gpu_quantize(inp)
    q = to_dev(inp.q)
    wide = torch.zeros(q.shape[:2] + (2 * Hq, 128), dtype=q.dtype, device=q.device)
    wide[:, :, ::2] = q
    qv = wide[:, :, ::2]  # the same values through strides (element stride of a head: 256)
    for dt in (torch.float32, torch.bfloat16):
        ref, rl = mx.attn_fwd_fused(g["qc"], g["qs"], g["kc"], g["ks"], g["vc"], g["vcs"], g["vt"], g["vta"],
                                    inp.workload.scale, out_dtype=dt, layout=layout)
        for qq in (q, qv):
            got, gl = mx.attn_fwd_fused_bf16q(qq, g["kc"], g["ks"], g["vc"], g["vcs"], g["vt"], g["vta"],
                                              inp.workload.scale, out_dtype=dt, layout=layout)
            torch.cuda.synchronize()
            assert torch.equal(got, ref) and torch.equal(gl, rl)


def test_causality_every_t_tiny():
    """Perturbing every token after t (with a x64 V outlier at t+1) leaves GPU rows 0..t
    bit-identical, for every t of the tiny workload."""
    inp = make_inputs("tiny_s128")
    q, k, v = (to_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    o0, l0 = mx.attn_fwd(q, k, v, out_dtype=torch.float32)
    for t in range(127):
        p = perturb_after(inp, t, outlier_at_next=True)
        o1, l1 = mx.attn_fwd(to_dev(p.q), to_dev(p.k), to_dev(p.v), out_dtype=torch.float32)
        assert torch.equal(o0[:, :t + 1], o1[:, :t + 1]), t
        assert torch.equal(l0[:, :, :t + 1], l1[:, :, :t + 1]), t


@pytest.mark.parametrize("name,ts", [("gqa16x4_s8k_outliers", [31, 32, 33, 4095, 8159, 8190]),
                                     ("mha16_s16k", [63, 8200, 16350]),
                                     ("gqa16x4_s32k_amplitudes", [40, 16383, 32700]),
                                     ("mha16_s32k_sbhd", [100, 20000, 32740])])
def test_causality_workloads(name, ts):
    inp = make_inputs(name)
    lay = inp.workload.layout
    q, k, v = (to_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    o0, l0 = mx.attn_fwd(q, k, v, layout=lay, out_dtype=torch.float32)
    rows = (lambda o, t: o[:, :t + 1]) if lay == "bshd" else (lambda o, t: o[:t + 1])
    for t in ts:
        say(f"causality {name} t={t}")
        p = perturb_after(inp, t, outlier_at_next=True)
        o1, l1 = mx.attn_fwd(to_dev(p.q), to_dev(p.k), to_dev(p.v), layout=lay, out_dtype=torch.float32)
        assert torch.equal(rows(o0, t), rows(o1, t)), t
        assert torch.equal(l0[:, :, :t + 1], l1[:, :, :t + 1]), t
        # and the rows after t did change (the perturbation reached the kernel)
        assert not torch.equal(o0, o1), t


def test_deterministic_and_poison_overwritten():
    inp = make_inputs(custom(1, 8, 2, 1056, seed=13))
    q, k, v = (to_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    outs = []
    for _ in range(2):
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
        lse = torch.full((1, 8, 1056), float("nan"), dtype=torch.float32, device=q.device)
        ws = torch.full((mx.attn_fwd_workspace_bytes(1, 1056, 8, 2),), 0xFF, dtype=torch.uint8, device=q.device)
        mx.attn_fwd(q, k, v, out_dtype=torch.float32, workspace=ws, out=out, lse=lse)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any() and not torch.isnan(lse).any()
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_bshd_equals_sbhd():
    a = make_inputs(custom(2, 4, 2, 160, layout="bshd", seed=14))
    b = make_inputs(custom(2, 4, 2, 160, layout="sbhd", seed=14))
    oa, la = mx.attn_fwd(to_dev(a.q), to_dev(a.k), to_dev(a.v), layout="bshd", out_dtype=torch.float32)
    ob, lb = mx.attn_fwd(to_dev(b.q), to_dev(b.k), to_dev(b.v), layout="sbhd", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob.permute(1, 0, 2, 3)) and torch.equal(la, lb)


def test_gqa_equals_repeated_kv():
    inp = make_inputs(custom(1, 8, 2, 256, seed=15))
    q, k, v = (to_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    o1, l1 = mx.attn_fwd(q, k, v, out_dtype=torch.float32)
    k4 = k.repeat_interleave(4, dim=2).contiguous()
    v4 = v.repeat_interleave(4, dim=2).contiguous()
    o2, l2 = mx.attn_fwd(q, k4, v4, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_accuracy_against_unquantized(name):
    """Accuracy report (printed as one ACCURACY line per workload): on the sampled rows, max|err|/RMS
    and RMS(err)/RMS of (i) the GPU leak-free forward vs the oracle, (ii) the GPU leak-free forward vs
    the fp64 unquantised causal attention on the same bf16 inputs, (iii) the oracle's ordinary
    (leaky) causal MXFP8 forward vs that same reference. RMS is that of the unquantised output. The
    MXFP8 error against the unquantised reference is quantisation error, so (ii) is only checked to
    be of the size of the leaky variant's (iii), not against a tolerance."""
    inp = make_inputs(name)
    w = inp.workload
    say(f"accuracy {name}")
    go, _ = gpu_forward(inp, torch.float32)
    rows = None if w.S <= 1024 else sample_rows(w.S, w.seed)
    q, k, v = oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v")
    z = _oracle_quant(inp)
    ro, _, _ = oracle.forward(q, k, v, w.scale, rows, quant=z)
    rr, _ = oracle.attn_reference(q, k, v, w.scale, rows)
    rl, _ = oracle.forward_leaky(q, k, v, w.scale, rows, quant=z)
    rms = np.sqrt(np.mean(rr ** 2)) if rows is None else \
        np.sqrt(np.mean(oracle.attn_reference(q, k, v, w.scale, uniform_rows(w.S, w.seed))[0] ** 2))
    sel = slice(None) if rows is None else rows
    g = go[:, :, sel]
    fig = lambda e: (np.max(np.abs(e)) / rms, np.sqrt(np.mean(e ** 2)) / rms)
    e1, e2, e3 = fig(g - ro), fig(g - rr), fig(rl - rr)
    say(f"ACCURACY {name} rows={'all' if rows is None else len(rows)} rms_ref={rms:.4e} | "
        f"gpu-vs-oracle max {e1[0]:.3e} rms {e1[1]:.3e} | gpu-vs-unquantised max {e2[0]:.3e} rms {e2[1]:.3e} | "
        f"leaky-oracle-vs-unquantised max {e3[0]:.3e} rms {e3[1]:.3e}")
    assert e2[1] <= 2.0 * e3[1] + 1e-3
