"""The allocation-free forward entry point, mxfa_attn_fwd_noalloc, through the C ABI: on two calls in
a row (the second on a smaller problem, so the static workspace holds the first call's larger
contents), its output and LSE equal mxfa_attn_fwd's with a caller workspace bit for bit, and the
second call leaves the device's free memory unchanged (the first call on a device looks up the
static array's address, which is when the HIP runtime backs it). Named to be collected last."""
import numpy as np
import pytest
import torch

import causal_mxfp8_block_amd as mx
from causal_mxfp8_block_amd.inputs import custom, make_inputs
from gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, S, layout, values, seed, dtype):
    inp = make_inputs(custom(B, Hq, Hkv, S, layout=layout, values=values, seed=seed))
    q, k, v = (to_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    ref_o, ref_l = mx.attn_fwd(q, k, v, inp.workload.scale, layout=layout, out_dtype=dtype)
    out = torch.full(q.shape, float("nan"), dtype=dtype, device=q.device)
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    got_o, got_l = mx.attn_fwd_noalloc(q, k, v, inp.workload.scale, layout=layout, out=out, lse=lse)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    say(f"noalloc {B}x{Hq}/{Hkv}x{S} {layout} {dtype}: equal {torch.equal(got_o, ref_o)}, "
        f"free memory change {free1 - free0} bytes")
    assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l)
    return free1 - free0


def test_noalloc_equals_attn_fwd_on_two_calls():
    _case(1, 16, 4, 4096, "bshd", "token_amplitudes", 61, torch.float32)
    change = _case(2, 4, 2, 416, "sbhd", "outliers", 62, torch.bfloat16)
    assert change == 0


def test_noalloc_refuses_a_problem_larger_than_its_workspace():
    need = mx.attn_fwd_workspace_bytes(1, 65536, 16, 16)
    assert need > mx.NOALLOC_WORKSPACE_BYTES
    q = torch.empty((1, 64, 16, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(mx.MxfaError, match="static workspace"):
        L = mx.lib()
        mx._check(L.mxfa_attn_fwd_noalloc(q.data_ptr(), 65536 * 2048, 2048, 128, q.data_ptr(), 65536 * 2048, 2048,
                                          128, q.data_ptr(), 65536 * 2048, 2048, 128, 1, 65536, 16, 16, 128, 0.1,
                                          q.data_ptr(), 65536 * 2048, 2048, 128, 1, None, None))
