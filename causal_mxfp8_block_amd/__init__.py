"""Leak-free causal MXFP8 attention forward for AMD MI355X (gfx950).

A thin ctypes binding over libmxfa.so (C ABI in include/mxfa.h): it turns torch tensors into device
pointers and sizes, allocates outputs with torch and passes torch's current HIP stream. Every step of
the computation runs in the library's HIP kernels; there is no host or PyTorch fallback, and a
missing or unloadable library raises.

Method: TransformerEngine PR #3865, "[PyTorch] Add causal MXFP8 attention without future-token
leakage through V scales" (section "Description").
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxfa.so")
_lib = None

ROWWISE, V = 0, 1
OUT_BF16, OUT_F32 = 0, 1
NOALLOC_WORKSPACE_BYTES = 256 << 20  # MXFA_NOALLOC_WORKSPACE_BYTES of include/mxfa.h


class MxfaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"mxfa status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libmxfa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with causal_mxfp8_block_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.mxfa_status_string.argtypes = [I]
        L.mxfa_status_string.restype = ctypes.c_char_p
        L.mxfa_last_error.argtypes = []
        L.mxfa_last_error.restype = ctypes.c_char_p
        L.mxfa_mxfp8_quantize.argtypes = [P, I, I, I, I, I64, I64, I64, I, P, P, P, P, P]
        L.mxfa_mxfp8_quantize.restype = I
        L.mxfa_mxfp8_quantize_kv.argtypes = [P, I64, I64, I64] * 2 + [I, I, I, I] + [P] * 7
        L.mxfa_mxfp8_quantize_kv.restype = I
        six = [P] * 6
        L.mxfa_attn_fwd_completed_blocks.argtypes = six + [I, I, I, I, I, F, P, P, P]
        L.mxfa_attn_fwd_completed_blocks.restype = I
        L.mxfa_attn_fwd_own_block.argtypes = six + [I, I, I, I, I, F, P, P, P]
        L.mxfa_attn_fwd_own_block.restype = I
        L.mxfa_lse_merge.argtypes = [P, P, P, P, I, I, I, I, P, I64, I64, I64, I, P, P]
        L.mxfa_lse_merge.restype = I
        L.mxfa_attn_fwd_fused.argtypes = [P] * 8 + [I, I, I, I, I, F, P, I64, I64, I64, I, P, P]
        L.mxfa_attn_fwd_fused.restype = I
        L.mxfa_attn_fwd_fused_mxfp8.argtypes = [P] * 8 + [I, I, I, I, I, F, P, I64, I64, I64, P, P, P]
        L.mxfa_attn_fwd_fused_mxfp8.restype = I
        L.mxfa_attn_fwd_fused_bf16q.argtypes = [P, I64, I64, I64] + [P] * 6 + [I, I, I, I, I, F, P, I64, I64, I64, I,
                                                                         P, P]
        L.mxfa_attn_fwd_fused_bf16q.restype = I
        L.mxfa_attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
        L.mxfa_attn_bwd_workspace_bytes.restype = SZ
        L.mxfa_attn_bwd.argtypes = six + [P, P, P, I, I, I, I, I, F, I64, I64, I64, I64, I64, I64, P, SZ, P, P, P, P]
        L.mxfa_attn_bwd.restype = I
        L.mxfa_attn_fwd_leaky.argtypes = six + [I, I, I, I, I, F, P, I64, I64, I64, I, P, P]
        L.mxfa_attn_fwd_leaky.restype = I
        L.mxfa_attn_fwd_workspace_bytes.argtypes = [I, I, I, I, I]
        L.mxfa_attn_fwd_workspace_bytes.restype = SZ
        L.mxfa_attn_fwd.argtypes = [P, I64, I64, I64] * 3 + [I, I, I, I, I, F, P, SZ, P, I64, I64, I64, I, P, P]
        L.mxfa_attn_fwd.restype = I
        L.mxfa_attn_fwd_noalloc.argtypes = [P, I64, I64, I64] * 3 + [I, I, I, I, I, F, P, I64, I64, I64, I, P, P]
        L.mxfa_attn_fwd_noalloc.restype = I
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise MxfaError(status, lib().mxfa_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _p(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def view_of(x: torch.Tensor, layout: str) -> tuple[int, int, int, int, int, int, int]:
    """(B, S, H, D, sb, ss, sh) of a 4-D tensor stored as [B,S,H,D] ('bshd') or [S,B,H,D] ('sbhd')."""
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("expected a 4-D tensor with unit stride along D")
    if layout == "bshd":
        B, S, H, D = x.shape
        return B, S, H, D, x.stride(0), x.stride(1), x.stride(2)
    if layout == "sbhd":
        S, B, H, D = x.shape
        return B, S, H, D, x.stride(1), x.stride(0), x.stride(2)
    raise ValueError(f"unknown layout {layout!r}")


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def mxfp8_quantize(x: torch.Tensor, mode: str = "rowwise", layout: str = "bshd", v_outputs: str = "both"):
    """MXFP8-encode a bf16 tensor.

    rowwise: returns (codes [B,H,S,D] u8, scales [B,H,S,D/32] u8) -- Q and K.
    v:       returns (col_codes [B,H,D,S], col_scales [B,H,S/32,D], tn_codes [B,H,S,D], tn_amps [B,H,S]);
             ``v_outputs`` = "col" or "tn" skips the other pair (returned as None).
    """
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    B, S, H, D, sb, ss, sh = view_of(x, layout)
    kw = dict(dtype=torch.uint8, device=x.device)
    if mode == "rowwise":
        codes = torch.empty((B, H, S, D), **kw)
        scales = torch.empty((B, H, S, D // 32), **kw)
        _check(lib().mxfa_mxfp8_quantize(_p(x), B, S, H, D, sb, ss, sh, ROWWISE, _p(codes), _p(scales), None, None,
                                         _stream(x)))
        return codes, scales
    if mode == "v":
        col = v_outputs in ("both", "col")
        tn = v_outputs in ("both", "tn")
        cc = torch.empty((B, H, D, S), **kw) if col else None
        cs = torch.empty((B, H, S // 32, D), **kw) if col else None
        tc = torch.empty((B, H, S, D), **kw) if tn else None
        ta = torch.empty((B, H, S), **kw) if tn else None
        _check(lib().mxfa_mxfp8_quantize(_p(x), B, S, H, D, sb, ss, sh, V, _p(cc), _p(cs), _p(tc), _p(ta), _stream(x)))
        return cc, cs, tc, ta
    raise ValueError(f"unknown mode {mode!r}")


def mxfp8_quantize_kv(k: torch.Tensor, v: torch.Tensor, layout: str = "bshd"):
    """K (rowwise) and V (both forms) in one launch, the bytes of mxfp8_quantize(k, "rowwise") and
    mxfp8_quantize(v, "v"): returns (k_codes, k_scales, v_codes, v_scales, v_tn_codes, v_tn_amps)."""
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("k and v must be bfloat16")
    B, S, H, D, ksb, kss, ksh = view_of(k, layout)
    vB, vS, vH, vD, vsb, vss, vsh = view_of(v, layout)
    if (vB, vS, vH, vD) != (B, S, H, D):
        raise ValueError("k and v must have the same shape")
    kw = dict(dtype=torch.uint8, device=k.device)
    kc, ks = torch.empty((B, H, S, D), **kw), torch.empty((B, H, S, D // 32), **kw)
    vc, vcs = torch.empty((B, H, D, S), **kw), torch.empty((B, H, S // 32, D), **kw)
    vt, vta = torch.empty((B, H, S, D), **kw), torch.empty((B, H, S), **kw)
    _check(lib().mxfa_mxfp8_quantize_kv(_p(k), ksb, kss, ksh, _p(v), vsb, vss, vsh, B, S, H, D, _p(kc), _p(ks),
                                        _p(vc), _p(vcs), _p(vt), _p(vta), _stream(k)))
    return kc, ks, vc, vcs, vt, vta


def attn_fwd_completed_blocks(qc, qs, kc, ks, vc, vcs, softmax_scale: float | None = None, o_c=None, lse_c=None):
    """Completed-block partial: (o_c fp32 [B,Hq,S,D], lse_c fp32 [B,Hq,S])."""
    B, Hq, S, D = qc.shape
    Hkv = kc.shape[1]
    scale = default_scale(D) if softmax_scale is None else softmax_scale
    if o_c is None:
        o_c = torch.empty((B, Hq, S, D), dtype=torch.float32, device=qc.device)
    if lse_c is None:
        lse_c = torch.empty((B, Hq, S), dtype=torch.float32, device=qc.device)
    _check(lib().mxfa_attn_fwd_completed_blocks(_p(qc), _p(qs), _p(kc), _p(ks), _p(vc), _p(vcs), B, S, Hq, Hkv, D,
                                                scale, _p(o_c), _p(lse_c), _stream(qc)))
    return o_c, lse_c


def attn_fwd_own_block(qc, qs, kc, ks, vt, vta, softmax_scale: float | None = None, o_o=None, lse_o=None):
    """Own-block partial on the token-normalised V: (o_o fp32 [B,Hq,S,D], lse_o fp32 [B,Hq,S])."""
    B, Hq, S, D = qc.shape
    Hkv = kc.shape[1]
    scale = default_scale(D) if softmax_scale is None else softmax_scale
    if o_o is None:
        o_o = torch.empty((B, Hq, S, D), dtype=torch.float32, device=qc.device)
    if lse_o is None:
        lse_o = torch.empty((B, Hq, S), dtype=torch.float32, device=qc.device)
    _check(lib().mxfa_attn_fwd_own_block(_p(qc), _p(qs), _p(kc), _p(ks), _p(vt), _p(vta), B, S, Hq, Hkv, D, scale,
                                         _p(o_o), _p(lse_o), _stream(qc)))
    return o_o, lse_o


def _out_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return OUT_BF16
    if dtype == torch.float32:
        return OUT_F32
    raise TypeError("output dtype must be bfloat16 or float32")


def lse_merge(o_c, lse_c, o_o, lse_o, out_dtype=torch.bfloat16, layout: str = "bshd", out=None, lse=None):
    """Merge the partials: (out [B,S,H,D] or [S,B,H,D] in out_dtype, lse fp32 [B,H,S])."""
    B, H, S, D = o_c.shape
    if out is None:
        shape = (B, S, H, D) if layout == "bshd" else (S, B, H, D)
        out = torch.empty(shape, dtype=out_dtype, device=o_c.device)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=o_c.device)
    _, _, _, _, osb, oss, osh = view_of(out, layout)
    _check(lib().mxfa_lse_merge(_p(o_c), _p(lse_c), _p(o_o), _p(lse_o), B, S, H, D, _p(out), osb, oss, osh,
                                _out_code(out.dtype), _p(lse), _stream(o_c)))
    return out, lse


def attn_fwd_fused(qc, qs, kc, ks, vc, vcs, vt, vta, softmax_scale: float | None = None, out_dtype=torch.bfloat16,
                   layout: str = "bshd", out=None, lse=None):
    """Both partials and the merge in one kernel, from the codes: (out in ``layout``, lse [B,Hq,S])."""
    B, Hq, S, D = qc.shape
    Hkv = kc.shape[1]
    scale = default_scale(D) if softmax_scale is None else softmax_scale
    if out is None:
        shape = (B, S, Hq, D) if layout == "bshd" else (S, B, Hq, D)
        out = torch.empty(shape, dtype=out_dtype, device=qc.device)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=qc.device)
    _, _, _, _, osb, oss, osh = view_of(out, layout)
    _check(lib().mxfa_attn_fwd_fused(_p(qc), _p(qs), _p(kc), _p(ks), _p(vc), _p(vcs), _p(vt), _p(vta), B, S, Hq, Hkv,
                                     D, scale, _p(out), osb, oss, osh, _out_code(out.dtype), _p(lse), _stream(qc)))
    return out, lse


def attn_fwd_fused_bf16q(q, kc, ks, vc, vcs, vt, vta, softmax_scale: float | None = None, out_dtype=torch.bfloat16,
                         layout: str = "bshd", out=None, lse=None):
    """The fused forward with Q as bf16 (``layout`` view), quantised inside the attention kernel:
    (out in ``layout``, lse [B,Hq,S]); equal to mxfp8_quantize(q) followed by attn_fwd_fused."""
    B, S, Hq, D, qsb, qss, qsh = view_of(q, layout)
    Hkv = kc.shape[1]
    scale = default_scale(D) if softmax_scale is None else softmax_scale
    if out is None:
        shape = (B, S, Hq, D) if layout == "bshd" else (S, B, Hq, D)
        out = torch.empty(shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _, _, _, _, osb, oss, osh = view_of(out, layout)
    _check(lib().mxfa_attn_fwd_fused_bf16q(_p(q), qsb, qss, qsh, _p(kc), _p(ks), _p(vc), _p(vcs), _p(vt), _p(vta), B,
                                           S, Hq, Hkv, D, scale, _p(out), osb, oss, osh, _out_code(out.dtype),
                                           _p(lse), _stream(q)))
    return out, lse


def attn_fwd_fused_mxfp8(qc, qs, kc, ks, vc, vcs, vt, vta, softmax_scale: float | None = None,
                         layout: str = "bshd"):
    """The fused forward with an MXFP8 output: (E4M3 codes u8 in ``layout`` [B,S,Hq,D] or [S,B,Hq,D],
    E8M0 bytes u8 [B,Hq,S,D/32], lse [B,Hq,S])."""
    B, Hq, S, D = qc.shape
    Hkv = kc.shape[1]
    scale = default_scale(D) if softmax_scale is None else softmax_scale
    shape = (B, S, Hq, D) if layout == "bshd" else (S, B, Hq, D)
    codes = torch.empty(shape, dtype=torch.uint8, device=qc.device)
    sf_o = torch.empty((B, Hq, S, D // 32), dtype=torch.uint8, device=qc.device)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=qc.device)
    _, _, _, _, osb, oss, osh = view_of(codes, layout)
    _check(lib().mxfa_attn_fwd_fused_mxfp8(_p(qc), _p(qs), _p(kc), _p(ks), _p(vc), _p(vcs), _p(vt), _p(vta), B, S, Hq,
                                           Hkv, D, scale, _p(codes), osb, oss, osh, _p(sf_o), _p(lse), _stream(qc)))
    return codes, sf_o, lse


def attn_fwd_leaky(qc, qs, kc, ks, vc, vcs, softmax_scale: float | None = None, out_dtype=torch.bfloat16,
                   layout: str = "bshd", out=None, lse=None):
    """Ordinary causal MXFP8 (leaks through V scales; for comparison): (out in ``layout``, lse [B,Hq,S])."""
    B, Hq, S, D = qc.shape
    Hkv = kc.shape[1]
    scale = default_scale(D) if softmax_scale is None else softmax_scale
    if out is None:
        shape = (B, S, Hq, D) if layout == "bshd" else (S, B, Hq, D)
        out = torch.empty(shape, dtype=out_dtype, device=qc.device)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=qc.device)
    _, _, _, _, osb, oss, osh = view_of(out, layout)
    _check(lib().mxfa_attn_fwd_leaky(_p(qc), _p(qs), _p(kc), _p(ks), _p(vc), _p(vcs), B, S, Hq, Hkv, D, scale, _p(out),
                                     osb, oss, osh, _out_code(out.dtype), _p(lse), _stream(qc)))
    return out, lse


def attn_fwd_workspace_bytes(B: int, S: int, Hq: int, Hkv: int, D: int = 128) -> int:
    return int(lib().mxfa_attn_fwd_workspace_bytes(B, S, Hq, Hkv, D))


def attn_fwd(q, k, v, softmax_scale: float | None = None, layout: str = "bshd", out_dtype=torch.bfloat16,
             workspace=None, out=None, lse=None):
    """The whole leak-free forward in one call: K quantised rowwise and V columnwise plus
    token-normalised into the workspace, then the fused attention kernel, which quantises Q itself
    (rowwise, the same codes and scales as mxfp8_quantize) and writes O and the LSE.

    q [B,S,Hq,D], k and v [B,S,Hkv,D] bf16 in ``layout``; returns (out in q's layout, lse [B,Hq,S])."""
    B, S, Hq, D, qsb, qss, qsh = view_of(q, layout)
    _, _, Hkv, _, ksb, kss, ksh = view_of(k, layout)
    _, _, _, _, vsb, vss, vsh = view_of(v, layout)
    scale = default_scale(D) if softmax_scale is None else softmax_scale
    need = attn_fwd_workspace_bytes(B, S, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _, _, _, _, osb, oss, osh = view_of(out, layout)
    _check(lib().mxfa_attn_fwd(_p(q), qsb, qss, qsh, _p(k), ksb, kss, ksh, _p(v), vsb, vss, vsh, B, S, Hq, Hkv, D,
                               scale, _p(workspace), workspace.numel(), _p(out), osb, oss, osh,
                               _out_code(out.dtype), _p(lse), _stream(q)))
    return out, lse


def attn_fwd_noalloc(q, k, v, softmax_scale: float | None = None, layout: str = "bshd", out_dtype=torch.bfloat16,
                     out=None, lse=None):
    """attn_fwd through the entry point that allocates nothing (its workspace is the library's static
    device array; calls that overlap on one device race). The outputs are allocated here unless
    given; returns (out in q's layout, lse [B,Hq,S])."""
    B, S, Hq, D, qsb, qss, qsh = view_of(q, layout)
    _, _, Hkv, _, ksb, kss, ksh = view_of(k, layout)
    _, _, _, _, vsb, vss, vsh = view_of(v, layout)
    scale = default_scale(D) if softmax_scale is None else softmax_scale
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _, _, _, _, osb, oss, osh = view_of(out, layout)
    _check(lib().mxfa_attn_fwd_noalloc(_p(q), qsb, qss, qsh, _p(k), ksb, kss, ksh, _p(v), vsb, vss, vsh, B, S, Hq,
                                       Hkv, D, scale, _p(out), osb, oss, osh, _out_code(out.dtype), _p(lse),
                                       _stream(q)))
    return out, lse


def attn_bwd(qc, qs, kc, ks, vt, vta, o, lse, do, softmax_scale: float | None = None, layout: str = "bshd",
             workspace=None):
    """Backward on decoded operands: (dq like ``o``, dk, dv [B,S,Hkv,D] (or [S,B,Hkv,D]) bf16).

    o and do are the forward's output and its gradient, bf16 in ``layout``; lse the forward's [B,Hq,S]."""
    B, Hq, S, D = qc.shape
    Hkv = kc.shape[1]
    scale = default_scale(D) if softmax_scale is None else softmax_scale
    if do.stride() != o.stride():
        do = do.contiguous() if o.is_contiguous() else torch.empty_like(o).copy_(do)
    dq = torch.empty_like(o)
    kshape = (B, S, Hkv, D) if layout == "bshd" else (S, B, Hkv, D)
    dk = torch.empty(kshape, dtype=torch.bfloat16, device=qc.device)
    dv = torch.empty(kshape, dtype=torch.bfloat16, device=qc.device)
    need = int(lib().mxfa_attn_bwd_workspace_bytes(B, S, Hq, Hkv, D))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=qc.device)
    _, _, _, _, qsb, qss, qsh = view_of(o, layout)
    _, _, _, _, ksb, kss, ksh = view_of(dk, layout)
    _check(lib().mxfa_attn_bwd(_p(qc), _p(qs), _p(kc), _p(ks), _p(vt), _p(vta), _p(o), _p(lse), _p(do), B, S, Hq,
                               Hkv, D, scale, qsb, qss, qsh, ksb, kss, ksh, _p(workspace), workspace.numel(), _p(dq),
                               _p(dk), _p(dv), _stream(qc)))
    return dq, dk, dv

