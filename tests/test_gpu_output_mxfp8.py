"""GPU block-scaled (MXFP8) output of the fused forward, attn_fwd_fused_mxfp8: the E4M3 codes and
E8M0 bytes equal, bit for bit, the oracle's MXFP8 encoding (rules O1/O2 in blocks of 32 along D) of
the same kernel's fp32 output; the LSE equals the fp32 call's; and the decoded output stays within
half an E4M3 step of the oracle's leak-free output plus the parity gate."""
import numpy as np
import pytest
import torch

import oracle
import causal_mxfp8_block_amd as mx
from causal_mxfp8_block_amd.inputs import custom, make_inputs
from gpu_helpers import gpu_quantize, oracle_view, say

pytestmark = pytest.mark.gpu


def _run(inp):
    w = inp.workload
    g = gpu_quantize(inp)
    args = (g["qc"], g["qs"], g["kc"], g["ks"], g["vc"], g["vcs"], g["vt"], g["vta"], w.scale)
    o32, l32 = mx.attn_fwd_fused(*args, out_dtype=torch.float32, layout=w.layout)
    codes, sf, l8 = mx.attn_fwd_fused_mxfp8(*args, layout=w.layout)
    torch.cuda.synchronize()
    to_bhsd = (lambda t: t.permute(0, 2, 1, 3)) if w.layout == "bshd" else (lambda t: t.permute(1, 2, 0, 3))
    return (to_bhsd(o32).double().cpu().numpy(), l32.cpu().numpy(), to_bhsd(codes).cpu().numpy(), sf.cpu().numpy(),
            l8.cpu().numpy())


@pytest.mark.parametrize("case", ["tiny", "small", "s8k"])
def test_mxfp8_output_is_the_encoding_of_the_fp32_output(case):
    if case == "tiny":
        inp = make_inputs("tiny_s128")
    elif case == "small":
        inp = make_inputs(custom(2, 4, 2, 416, values="outliers", seed=31))
    else:
        inp = make_inputs("gqa16x4_s8k_outliers")
    say(f"mxfp8 output {case}")
    o32, l32, codes, sf, l8 = _run(inp)
    rc, rs = oracle.quantize_rows(o32)
    assert np.array_equal(sf, rs)
    assert np.array_equal(codes, rc)
    assert np.array_equal(l8, l32)


def test_mxfp8_output_accuracy_small():
    """Decoded MXFP8 output vs the oracle's fp64 leak-free output: every element within half an E4M3
    step of the kernel's own fp32 output (the encoding's rounding), and within that step plus the
    forward parity gate's bound of the oracle (2e-2 * RMS, plus the R15 allowance where it applies)."""
    inp = make_inputs(custom(1, 2, 1, 256, values="normal", seed=32))
    w = inp.workload
    o32, _, codes, sf, _ = _run(inp)
    dec = np.vectorize(oracle.e4m3_decode)(codes.astype(np.int64)) * \
        np.ldexp(1.0, np.repeat(sf.astype(np.int64) - 127, 32, axis=-1))
    ro, _, parts = oracle.forward(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"), w.scale)
    k = np.repeat(sf.astype(np.int64) - 127, 32, axis=-1)
    # half the E4M3 spacing at |x| (2^-4 |x| for normals; 2^(k-10) on the subnormal grid)
    step = np.maximum(np.ldexp(np.abs(o32), -4), np.ldexp(1.0, k - 10))
    assert np.all(np.abs(dec - o32) <= step * (1 + 1e-9))
    rms = np.sqrt(np.mean(ro ** 2))
    excess = np.abs(dec - ro) - step - parts["allowance"]
    say(f"decoded MXFP8 output vs oracle: max|err|/rms = {np.max(np.abs(dec - ro)) / rms:.3e}, "
        f"max(|err| - step - allowance)/rms = {excess.max() / rms:.3e}")
    assert excess.max() <= 2e-2 * rms
