"""Seeded random problem shapes, beyond the fixed ones of the other tests: batch, head counts (MHA and
GQA groups of 2 to 8), sequence lengths that are any multiple of 32 (ragged against the 128-query
workgroups and the 64-key tiles), both layouts and the three value distributions. For each: the
whole forward (mxfa_attn_fwd) on every row against the oracle under the forward's gate
(max|err| <= 2e-2 * RMS beyond the allowance, see test_gpu_attention.py), and the own-block entry
point against the oracle's own-block partial within 1e-4 * RMS (exact scores, no quantised P)."""
import numpy as np
import pytest
import torch

import oracle
import causal_mxfp8_block_amd as mx
from causal_mxfp8_block_amd.inputs import custom, make_inputs
from gpu_helpers import gate, gpu_forward, gpu_quantize, oracle_view, report, say

pytestmark = pytest.mark.gpu
TOL = 2e-2
MAX_OVER = 2e-3


def _cases(n=10, seed=3):
    rng = np.random.default_rng(seed)
    heads = [(1, 1), (2, 1), (3, 3), (4, 2), (6, 2), (8, 1), (8, 4)]
    out = []
    for i in range(n):
        Hq, Hkv = heads[rng.integers(len(heads))]
        out.append(dict(B=int(rng.integers(1, 3)), Hq=Hq, Hkv=Hkv, S=32 * int(rng.integers(1, 25)),
                        layout=["bshd", "sbhd"][rng.integers(2)],
                        values=["normal", "outliers", "token_amplitudes"][rng.integers(3)], seed=100 + i))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"B{c['B']}_h{c['Hq']}x{c['Hkv']}_S{c['S']}_{c['layout']}_{c['values']}")
def test_random_shape_forward_and_own_block(case):
    w = custom(case["B"], case["Hq"], case["Hkv"], case["S"], layout=case["layout"], values=case["values"],
               seed=case["seed"])
    inp = make_inputs(w)
    say(f"random shape {case}")
    go, gl = gpu_forward(inp, torch.float32)
    z = oracle.quantize_all(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"))
    ro, rl, parts = oracle.forward(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"), w.scale,
                                   None, quant=z)
    rms = np.sqrt(np.mean(ro ** 2))
    gate("forward", go, ro, rms, None, allowance=parts["allowance"],
         allowance_hw=parts["allowance_code"] + parts["allowance_pv"], tol=TOL, max_over_frac=MAX_OVER)
    assert np.max(np.abs(gl - rl)) < 1e-3
    g = gpu_quantize(inp)
    oo, lo = mx.attn_fwd_own_block(g["qc"], g["qs"], g["kc"], g["ks"], g["vt"], g["vta"], w.scale)
    torch.cuda.synchronize()
    roo, rlo = oracle.attn_own(z.qc, z.qs, z.kc, z.ks, z.vt, z.vta, w.Hq, w.Hkv, w.scale)
    goo = oo.double().cpu().numpy()
    assert report("own block", goo, roo, np.sqrt(np.mean(roo ** 2))) <= 1e-4
    assert np.max(np.abs(lo.double().cpu().numpy() - rlo)) < 1e-4


def _bwd_cases(n=6, seed=7):
    rng = np.random.default_rng(seed)
    heads = [(1, 1), (2, 1), (3, 3), (4, 2), (4, 1), (6, 3)]
    out = []
    for i in range(n):
        Hq, Hkv = heads[rng.integers(len(heads))]
        out.append(dict(B=int(rng.integers(1, 3)), Hq=Hq, Hkv=Hkv, S=32 * int(rng.integers(1, 11)),
                        layout=["bshd", "sbhd"][i % 2], values=["normal", "outliers", "token_amplitudes"][i % 3],
                        seed=200 + i))
    return out


@pytest.mark.parametrize("case", _bwd_cases(), ids=lambda c: f"B{c['B']}_h{c['Hq']}x{c['Hkv']}_S{c['S']}_{c['layout']}_{c['values']}")
def test_random_shape_backward(case):
    """attn_bwd on random shapes (both layouts, GQA sums, all value mixes) against the oracle's fp64
    backward, under the backward tests' gate (the R16 allowance plus the bf16 output rounding)."""
    from test_gpu_backward import TOL as BTOL, _dout, _gate, _gpu_bwd, _stats_from_oracle, _view
    w = custom(case["B"], case["Hq"], case["Hkv"], case["S"], layout=case["layout"], values=case["values"],
               seed=case["seed"])
    inp = make_inputs(w)
    say(f"random backward {case}")
    z = oracle.quantize_all(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"))
    obits, lse = _stats_from_oracle(inp, z)
    gbits = _dout(inp, case["seed"] + 1)
    dq, dk, dv = _gpu_bwd(inp, obits, lse, gbits)
    rq, rk, rv, aq, ak, av = oracle.attn_bwd(z.qc, z.qs, z.kc, z.ks, z.vt, z.vta, _view(obits, w.layout), lse,
                                             _view(gbits, w.layout), w.scale, allowance=True)
    for name, got, ref, al in (("dq", dq, rq, aq), ("dk", dk, rk, ak), ("dv", dv, rv, av)):
        assert _gate(f"{name}", got, ref, al) <= BTOL


@pytest.mark.parametrize("case", _cases(n=4, seed=11),
                         ids=lambda c: f"B{c['B']}_h{c['Hq']}x{c['Hkv']}_S{c['S']}_{c['layout']}_{c['values']}")
def test_random_shape_leaky(case):
    """The ordinary causal MXFP8 variant on random shapes against the oracle's leaky variant, under the
    same gate (both half-tile positions of the own block occur)."""
    from test_gpu_leaky import MAX_OVER as LMAX, TOL as LTOL, _gpu_leaky, _oracle_leaky
    w = custom(case["B"], case["Hq"], case["Hkv"], case["S"], layout=case["layout"], values=case["values"],
               seed=case["seed"])
    inp = make_inputs(w)
    say(f"random leaky {case}")
    go, gl, _ = _gpu_leaky(inp)
    ro, rl, A = _oracle_leaky(inp)
    rms = np.sqrt(np.mean(ro ** 2))
    gate("leaky", go, ro, rms, allowance=A.total, allowance_hw=A.code + A.pv, tol=LTOL, max_over_frac=LMAX)
    assert np.max(np.abs(gl - rl)) < 1e-3
