"""Edge cases of the attention kernels on the GPU, through the C ABI:

* every E4M3 code of the token-normalised V decodes exactly (the own-block kernel and the fused
  epilogue decode V with the hardware conversion): query 0 of a sequence sees only key 0, so its
  output row is key 0's decoded row times its amplitude, bit for bit;
* a query whose running maximum lies far above the scores of a later key tile, in a wave where
  another query's maximum rises by more than the lazy-rescale threshold in that tile: its output
  stays finite and meets the oracle (the running exponent only ever rises after the first tile).
"""
import numpy as np
import pytest
import torch

import causal_mxfp8_block_amd as mx
import oracle
from causal_mxfp8_block_amd.inputs import bf16_bits, custom, make_inputs
from gpu_helpers import gate, say, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c - 1, c).astype(np.uint8)  # no NaN code


def test_every_e4m3_code_decodes_exactly():
    rng = np.random.default_rng(90)
    B, H, S = 2, 1, 64
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    qc, kc = _rand_codes(rng, (B, H, S, 128)), _rand_codes(rng, (B, H, S, 128))
    qs = rng.integers(118, 124, size=(B, H, S, 4)).astype(np.uint8)
    ks = rng.integers(118, 124, size=(B, H, S, 4)).astype(np.uint8)
    vt = _rand_codes(rng, (B, H, S, 128))
    all_codes = np.arange(256, dtype=np.uint8)
    all_codes = np.where((all_codes & 0x7F) == 0x7F, all_codes - 1, all_codes).astype(np.uint8)
    vt[0, 0, 0] = all_codes[:128]
    vt[1, 0, 0] = all_codes[128:]
    vta = rng.integers(120, 134, size=(B, H, S)).astype(np.uint8)
    vta[0, 0, 0], vta[1, 0, 0] = 127, 131
    vc = _rand_codes(rng, (B, H, 128, S))
    vcs = rng.integers(120, 130, size=(B, H, S // 32, 128)).astype(np.uint8)
    want = np.array([[oracle.e4m3_decode(int(c)) * 2.0 ** (int(vta[b, 0, 0]) - 127) for c in vt[b, 0, 0]]
                     for b in range(B)])
    g = {n: t(a) for n, a in dict(qc=qc, qs=qs, kc=kc, ks=ks, vc=vc, vcs=vcs, vt=vt, vta=vta).items()}
    oo, lo = mx.attn_fwd_own_block(g["qc"], g["qs"], g["kc"], g["ks"], g["vt"], g["vta"])
    of, lf = mx.attn_fwd_fused(g["qc"], g["qs"], g["kc"], g["ks"], g["vc"], g["vcs"], g["vt"], g["vta"],
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    got_own = oo[:, 0, 0].double().cpu().numpy()
    got_fused = of[:, 0, 0].double().cpu().numpy()  # [B,S,H,D]: row 0, head 0
    say(f"decode: own-block differs at {int(np.sum(got_own != want))}, fused at {int(np.sum(got_fused != want))} "
        f"of {want.size} codes")
    assert np.array_equal(got_own, want)
    assert np.array_equal(got_fused, want)


def test_running_exponent_never_scaled_up():
    """Row 170 has one huge score (key 0: its q equals key 0's k, both of magnitude 4 in every
    dimension); in the next key tile row 161 of the same wave meets a key whose score is about 60
    log2 units above its earlier maximum, which makes the wave raise its exponents. Row 170's scores
    in that tile lie about 250 log2 units below its own exponent."""
    inp = make_inputs(custom(1, 1, 1, 256, seed=91))
    q = inp.q.copy()
    k = inp.k.copy()
    u = np.where(np.arange(128) < 64, 4.0, -4.0).astype(np.float32)
    q[0, 170, 0] = bf16_bits(u)
    k[0, 0, 0] = bf16_bits(u)
    q[0, 161, 0] = bf16_bits(np.full(128, 2.0, np.float32))
    k[0, 100, 0] = bf16_bits(np.full(128, 2.0, np.float32))
    scale = inp.workload.scale
    out, lse = mx.attn_fwd(to_dev(q), to_dev(k), to_dev(inp.v), scale, out_dtype=torch.float32)
    z = oracle.quantize_all(q, k, inp.v)
    oc_g, lc_g = mx.attn_fwd_completed_blocks(*(torch.from_numpy(a).to(DEV) for a in (z.qc, z.qs, z.kc, z.ks, z.vc,
                                                                                        z.vcs)), scale)
    torch.cuda.synchronize()
    go = out.double().cpu().numpy().transpose(0, 2, 1, 3)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(lse.cpu().numpy()))
    assert np.all(np.isfinite(oc_g.cpu().numpy()))
    ro, rl, parts = oracle.forward(q, k, inp.v, scale, quant=z)
    rms = np.sqrt(np.mean(ro ** 2))
    gate("large score gap", go, ro, rms, allowance=parts["allowance"],
         allowance_hw=parts["allowance_code"] + parts["allowance_pv"], tol=2e-2, max_over_frac=2e-3)
    assert np.max(np.abs(lse.double().cpu().numpy() - rl)) < 1e-3
