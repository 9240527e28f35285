"""GPU ordinary ("leaky") causal MXFP8 attention, attn_fwd_leaky: parity with the oracle's leaky
variant, and the leak itself on the GPU: a later token of a query's own 32-token block changes that
query's output here, while the leak-free forward stays bit-identical.

Tolerance: as for the leak-free forward (gpu_helpers.gate): max|err| <= 2e-2 * RMS(oracle output)
except where the oracle's R15 allowance names an alternative valid P code under the hardware's
error bound, the excess within the allowance, at most 2e-3 of the elements over the plain
tolerance."""
import numpy as np
import pytest
import torch

import oracle
import causal_mxfp8_block_amd as mx
from causal_mxfp8_block_amd.inputs import custom, make_inputs, perturb_after
from gpu_helpers import gate, gpu_forward, gpu_quantize, oracle_view, sample_rows, say, uniform_rows

pytestmark = pytest.mark.gpu
TOL = 2e-2
MAX_OVER = 2e-3


def _gpu_leaky(inp, out_dtype=torch.float32):
    w = inp.workload
    g = gpu_quantize(inp)
    out, lse = mx.attn_fwd_leaky(g["qc"], g["qs"], g["kc"], g["ks"], g["vc"], g["vcs"], w.scale, out_dtype=out_dtype,
                                 layout=w.layout)
    torch.cuda.synchronize()
    o = out.float()
    o = o.permute(0, 2, 1, 3) if w.layout == "bshd" else o.permute(1, 2, 0, 3)
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), out


def _oracle_leaky(inp, rows=None):
    z = oracle.quantize_all(oracle_view(inp, "q"), oracle_view(inp, "k"), oracle_view(inp, "v"))
    w = inp.workload
    return oracle.attn_leaky(z.qc, z.qs, z.kc, z.ks, z.vc, z.vcs, w.Hq, w.Hkv, w.scale, rows, allowance=True)


@pytest.mark.parametrize("shape", [(1, 1, 1, 128), (2, 4, 2, 416), (1, 8, 2, 288), (1, 2, 1, 32), (1, 3, 1, 96),
                                   (1, 4, 2, 352)])
def test_leaky_matches_oracle_small(shape):
    """Every row of shapes spanning several query tiles, ragged tails, GQA and batch > 1 (both own-block
    positions in a 64-key tile occur)."""
    B, Hq, Hkv, S = shape
    inp = make_inputs(custom(B, Hq, Hkv, S, values="outliers", seed=100 + sum(shape)))
    say(f"leaky {shape}")
    go, gl, _ = _gpu_leaky(inp)
    ro, rl, A = _oracle_leaky(inp)
    rms = np.sqrt(np.mean(ro ** 2))
    gate("leaky", go, ro, rms, allowance=A.total, allowance_hw=A.code + A.pv, tol=TOL, max_over_frac=MAX_OVER)
    assert np.max(np.abs(gl - rl)) < 1e-3


@pytest.mark.parametrize("name", ["gqa16x4_s8k_outliers", "mha16_s32k_sbhd"])
def test_leaky_matches_oracle_workloads(name):
    inp = make_inputs(name)
    w = inp.workload
    say(f"leaky {name}")
    go, gl, _ = _gpu_leaky(inp)
    rows = sample_rows(w.S, w.seed)
    ro, rl, A = _oracle_leaky(inp, rows)
    ru = _oracle_leaky(inp, uniform_rows(w.S, w.seed))[0]
    rms = np.sqrt(np.mean(ru ** 2))
    gate(f"leaky {name}", go[:, :, rows], ro, rms, rows, allowance=A.total, allowance_hw=A.code + A.pv, tol=TOL,
         max_over_frac=MAX_OVER)
    assert np.max(np.abs(gl[:, :, rows] - rl)) < 1e-3


def test_leaky_bf16_is_rne_of_f32():
    inp = make_inputs(custom(1, 4, 2, 256, values="normal", seed=7))
    _, _, o32 = _gpu_leaky(inp, torch.float32)
    _, _, o16 = _gpu_leaky(inp, torch.bfloat16)
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_leak_is_visible_on_gpu_and_absent_from_leak_free():
    """Negative control on the GPU: with a x64 outlier planted at token t+1 and all tokens > t
    re-drawn, row t of the leaky output changes for t inside a 32-token block (at least half of the
    cases) and never at a block's last token; the leak-free forward's row t never changes."""
    inp = make_inputs("tiny_s128")
    base_leaky, _, _ = _gpu_leaky(inp)
    base_free, _ = gpu_forward(inp, torch.float32)
    changed, inside = 0, 0
    for t in range(0, 127):
        pert = perturb_after(inp, t, outlier_at_next=True)
        lk, _, _ = _gpu_leaky(pert)
        fr, _ = gpu_forward(pert, torch.float32)
        assert np.array_equal(fr[:, :, :t + 1], base_free[:, :, :t + 1]), t
        same = np.array_equal(lk[:, :, t], base_leaky[:, :, t])
        if t % 32 == 31:
            assert same, t  # t+1 opens a new block: nothing of t's blocks changed
        else:
            inside += 1
            changed += int(not same)
    say(f"leaky rows changed by a later token of their own block: {changed} of {inside}")
    assert changed >= inside // 2
