"""GPU parity of mxfp8_quantize against the oracle and brute force: bit-exact codes and scales."""
import numpy as np
import pytest
import torch

import blocks
import oracle
from causal_mxfp8_block_amd.inputs import WORKLOADS, make_inputs
from gpu_helpers import gpu_quantize, oracle_view, say, to_dev
import causal_mxfp8_block_amd as mx

pytestmark = pytest.mark.gpu


def test_rowwise_exhaustive_bf16():
    """Every finite bf16 value at every useful block exponent: codes and scales bit-exact."""
    blk, ks = blocks.exhaustive_blocks()
    x = blocks.as_rowwise_input(blk)
    say(f"rowwise exhaustive: {x.shape}")
    codes, scales = mx.mxfp8_quantize(to_dev(x), "rowwise")
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy().reshape(-1), (ks + 127).astype(np.uint8))
    got = codes.cpu().numpy().reshape(-1, 32)
    exp = blocks.expected_codes(blk, ks)
    bad = np.nonzero(np.any(got != exp, axis=1))[0]
    assert bad.size == 0, f"{bad.size} blocks differ, first {bad[:5]}"


def test_v_exhaustive_bf16():
    blk, ks = blocks.exhaustive_blocks()
    v = blocks.as_v_input(blk)
    say(f"v exhaustive: {v.shape}")
    cc, cs, tc, ta = mx.mxfp8_quantize(to_dev(v), "v")
    torch.cuda.synchronize()
    occ, ocs, otc, ota = oracle.quantize_v(v)
    assert np.array_equal(cc.cpu().numpy(), occ)
    assert np.array_equal(cs.cpu().numpy(), ocs)
    assert np.array_equal(tc.cpu().numpy(), otc)
    assert np.array_equal(ta.cpu().numpy(), ota)
    U = v.shape[1] // 32
    got = cc.cpu().numpy()[0, 0].reshape(128, U, 32).transpose(1, 0, 2).reshape(-1, 32)
    assert np.array_equal(got, blocks.expected_codes(blk, ks))


def test_v_outputs_subsets():
    inp = make_inputs("tiny_s128")
    v = to_dev(inp.v)
    cc, cs, tc, ta = mx.mxfp8_quantize(v, "v")
    c2, s2, t2, a2 = mx.mxfp8_quantize(v, "v", v_outputs="col")
    assert t2 is None and a2 is None and torch.equal(cc, c2) and torch.equal(cs, s2)
    c3, s3, t3, a3 = mx.mxfp8_quantize(v, "v", v_outputs="tn")
    assert c3 is None and s3 is None and torch.equal(tc, t3) and torch.equal(ta, a3)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_quantize_workloads_match_oracle(name):
    """Q, K (rowwise) and V (columnwise + token-normalised) of every benchmark workload."""
    inp = make_inputs(name)
    say(f"quantize workload {name}")
    g = {k: v.cpu().numpy() for k, v in gpu_quantize(inp).items()}
    qc, qs = oracle.quantize_rowwise(oracle_view(inp, "q"))
    kc, ks = oracle.quantize_rowwise(oracle_view(inp, "k"))
    vc, vcs, vt, vta = oracle.quantize_v(oracle_view(inp, "v"))
    for key, ref in dict(qc=qc, qs=qs, kc=kc, ks=ks, vc=vc, vcs=vcs, vt=vt, vta=vta).items():
        assert np.array_equal(g[key], ref), key


def test_quantize_ragged_and_strided():
    """S not a multiple of 128 (ragged V tile) and a non-contiguous head slice."""
    from causal_mxfp8_block_amd.inputs import custom
    inp = make_inputs(custom(2, 3, 3, 160, seed=31))
    full = to_dev(inp.q)  # [2,160,3,128]
    sl = full[:, :, 1:3, :]  # strided view: sh = 128, ss = 384
    c, s = mx.mxfp8_quantize(sl, "rowwise")
    ref_c, ref_s = oracle.quantize_rowwise(np.ascontiguousarray(inp.q[:, :, 1:3, :]))
    assert np.array_equal(c.cpu().numpy(), ref_c) and np.array_equal(s.cpu().numpy(), ref_s)
    out = mx.mxfp8_quantize(to_dev(inp.v), "v")
    ref = oracle.quantize_v(inp.v)
    for a, b in zip(out, ref):
        assert np.array_equal(a.cpu().numpy(), b)


@pytest.mark.parametrize("B,S,H,layout", [(1, 32, 1, "bshd"), (2, 96, 3, "bshd"), (1, 160, 4, "sbhd"),
                                          (1, 32768, 4, "bshd")])
def test_quantize_kv_equals_separate_calls_and_oracle(B, S, H, layout):
    """mxfp8_quantize_kv (one launch, what attn_fwd runs) = mxfp8_quantize(k, rowwise) and
    mxfp8_quantize(v, v) byte for byte, K and V from different strided views (token groups of 64 with
    a ragged last one at S = 96 and 160), and the oracle's encoders on the same inputs."""
    from causal_mxfp8_block_amd.inputs import custom
    inp = make_inputs(custom(B, 2 * H, H, S, layout=layout, values="token_amplitudes", seed=40 + S + H))
    say(f"quantize_kv B={B} S={S} H={H} {layout}")
    kfull, vfull = to_dev(inp.k), to_dev(inp.v)
    # K and V as views into wider tensors with different strides
    kwide = torch.zeros(kfull.shape[:-2] + (H + 1, 128), dtype=torch.bfloat16, device=kfull.device)
    kwide[..., 1:, :] = kfull
    k = kwide[..., 1:, :]
    got = mx.mxfp8_quantize_kv(k, vfull, layout)
    torch.cuda.synchronize()
    ref = list(mx.mxfp8_quantize(k, "rowwise", layout)) + list(mx.mxfp8_quantize(vfull, "v", layout))
    torch.cuda.synchronize()
    for name, a, b in zip(("kc", "ks", "vc", "vcs", "vt", "vta"), got, ref):
        assert torch.equal(a, b), name
    ok = oracle.quantize_rowwise(oracle_view(inp, "k")) + oracle.quantize_v(oracle_view(inp, "v"))
    for name, a, b in zip(("kc", "ks", "vc", "vcs", "vt", "vta"), got, ok):
        assert np.array_equal(a.cpu().numpy(), b), name
