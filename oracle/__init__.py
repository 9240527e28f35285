"""Plain fp64 CPU oracle for leak-free causal MXFP8 attention (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg
import this package; the product package never does, and the two share no code. The arithmetic
lives in ``oracle.c``; this module marshals numpy arrays and builds the library with gcc.

The method it models is TransformerEngine PR #3865 ("[PyTorch] Add causal MXFP8 attention without
future-token leakage through V scales", section "Description"): completed 32-key blocks in MXFP8
with columnwise V scales, the query's own block on a token-normalised V, merged through the
log-sum-exps.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP across rows, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h"))
    ):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, I64, F, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        lib.orc_e8m0_exponent.argtypes = [D]
        lib.orc_e8m0_exponent.restype = I
        lib.orc_e4m3_encode.argtypes = [D]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_decode.restype = D
        lib.orc_quantize_rowwise.argtypes = [P, I, I, I, I, I64, I64, I64, P, P]
        lib.orc_quantize_rows_f64.argtypes = [P, I64, I, P, P]
        lib.orc_attn_bwd_values.argtypes = [P] * 6 + [I, I, I, I, I, D, P, I, P, I, P, P, P, P, P, P]
        lib.orc_attn_bwd.argtypes = [P] * 7 + [I64, I64, I64, P, P, I64, I64, I64, I, I, I, I, I, F, P, I, P, I,
                                                P, P, P, P, P, P]
        lib.orc_quantize_v.argtypes = [P, I, I, I, I, I64, I64, I64, P, P, P, P]
        six = [P] * 6
        lib.orc_attn_completed.argtypes = six + [I, I, I, I, I, F, P, I, I, P, P, D, P, P, P, P, D, ctypes.c_uint64]
        lib.orc_attn_own.argtypes = six + [I, I, I, I, I, F, P, I, P, P, D, P, P, D, ctypes.c_uint64]
        lib.orc_attn_leaky.argtypes = six + [I, I, I, I, I, F, P, I, P, P, D, P, P, P, P, D, ctypes.c_uint64]
        lib.orc_lse_merge.argtypes = [P, P, P, P, I64, I, P, P]
        lib.orc_score_bound.argtypes = [P, P, P, P, I64, I64, P]
        raw = [P, I64, I64, I64] * 3
        lib.orc_attn_reference.argtypes = raw + [I, I, I, I, I, F, P, I, P, P]
        lib.orc_attn_identity.argtypes = raw + [I, I, I, I, I, F, P, I, P, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 0
    return a.ctypes.data


# ------------------------------------------------------------------------------- codec ---

def e8m0_exponent(amax: float) -> int:
    """O1: exponent k of the E8M0 scale of a block with maximum magnitude ``amax``."""
    return _load().orc_e8m0_exponent(float(amax))


def e4m3_encode(y: float) -> int:
    """O2: OCP E4M3FN code of ``y`` (nearest, ties to even, saturating, sign kept)."""
    return _load().orc_e4m3_encode(float(y))


def e4m3_decode(code: int) -> float:
    """O3: value of an E4M3 code."""
    return _load().orc_e4m3_decode(int(code))


# -------------------------------------------------------------------------- quantisers ---

@dataclass
class BF16View:
    """A bf16 tensor (uint16 bit patterns) with logical shape [B,S,H,D] and element strides."""
    data: np.ndarray  # the underlying uint16 buffer (any shape), C-contiguous
    B: int
    S: int
    H: int
    D: int
    sb: int
    ss: int
    sh: int

    @staticmethod
    def bshd(x: np.ndarray) -> "BF16View":
        B, S, H, D = x.shape
        x = np.ascontiguousarray(x)
        return BF16View(x, B, S, H, D, S * H * D, H * D, D)

    @staticmethod
    def sbhd(x: np.ndarray) -> "BF16View":
        """``x`` is stored [S,B,H,D]; the logical view is [B,S,H,D]."""
        S, B, H, D = x.shape
        x = np.ascontiguousarray(x)
        return BF16View(x, B, S, H, D, H * D, B * H * D, D)

    def logical(self) -> np.ndarray:
        """The logical [B,S,H,D] array (a copy)."""
        flat = self.data.reshape(-1)
        idx = (np.arange(self.B)[:, None, None, None] * self.sb + np.arange(self.S)[None, :, None, None] * self.ss
               + np.arange(self.H)[None, None, :, None] * self.sh + np.arange(self.D)[None, None, None, :])
        return flat[idx]


def _as_view(x) -> BF16View:
    if isinstance(x, BF16View):
        return x
    x = np.asarray(x)
    assert x.dtype == np.uint16 and x.ndim == 4
    return BF16View.bshd(x)


def quantize_rowwise(x) -> tuple[np.ndarray, np.ndarray]:
    """O4: rowwise MXFP8 codes [B,H,S,D] and scale bytes [B,H,S,D/32] of a bf16 [B,S,H,D] tensor."""
    v = _as_view(x)
    codes = np.empty((v.B, v.H, v.S, v.D), np.uint8)
    scales = np.empty((v.B, v.H, v.S, v.D // 32), np.uint8)
    _load().orc_quantize_rowwise(_ptr(v.data), v.B, v.S, v.H, v.D, v.sb, v.ss, v.sh, _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 of real-valued rows x [..., D] (blocks of 32 along D, rules O1/O2): (codes [..., D] u8,
    scales [..., D/32] u8). Used for the block-scaled output."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    D = x.shape[-1]
    n = x.size // D
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1] + (D // 32,), np.uint8)
    _load().orc_quantize_rows_f64(_ptr(x), n, D, _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_v(x) -> tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """O5 + O6: (col codes [B,H,D,S], col scales [B,H,S/32,D], tn codes [B,H,S,D], tn amplitudes [B,H,S])."""
    v = _as_view(x)
    cc = np.empty((v.B, v.H, v.D, v.S), np.uint8)
    cs = np.empty((v.B, v.H, v.S // 32, v.D), np.uint8)
    tc = np.empty((v.B, v.H, v.S, v.D), np.uint8)
    ta = np.empty((v.B, v.H, v.S), np.uint8)
    _load().orc_quantize_v(_ptr(v.data), v.B, v.S, v.H, v.D, v.sb, v.ss, v.sh, _ptr(cc), _ptr(cs), _ptr(tc),
                           _ptr(ta))
    return cc, cs, tc, ta


# --------------------------------------------------------------------------- attention ---

def _rows_arg(rows, S):
    if rows is None:
        return None, S
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < S))
    return r, int(r.size)


def _out(B, Hq, n, D):
    return np.empty((B, Hq, n, D), np.float64), np.empty((B, Hq, n), np.float64)


# Multiplier of the hardware error model of reading R15 (1: the gfx950 block-scaled FP8 MFMA as the
# probe tests measured it; 0: no hardware error, fp32 evaluation only).
HW_ERR = 1.0


def score_bound(ac, as_, bc, bs) -> np.ndarray:
    """Reading R15: bound [na, nb] of |hardware score - exact a.b| on the block-scaled FP8 MFMA for
    rows of codes ac [na,128] / scale bytes as_ [na,4] against bc [nb,128] / bs [nb,4]."""
    ac, as_, bc, bs = (np.ascontiguousarray(x, dtype=np.uint8) for x in (ac, as_, bc, bs))
    out = np.empty((ac.shape[0], bc.shape[0]))
    _load().orc_score_bound(_ptr(ac), _ptr(as_), _ptr(bc), _ptr(bs), ac.shape[0], bc.shape[0], _ptr(out))
    return out


@dataclass
class Allowance:
    """Reading R15 per output element [B,Hq,n,D]: ``total``, the largest change a kernel on the
    block-scaled FP8 MFMA can make; ``code``, its term (i), alternative valid P codes; ``pv``, its
    term (iii), the P.V products the MFMA cuts (the rest is the normaliser, own-block and
    merge-weight terms); and ``lse_err`` [B,Hq,n], the bound of the lse error."""
    total: np.ndarray
    code: np.ndarray
    pv: np.ndarray
    lse_err: np.ndarray


def _completed_like(fn, qc, qs, kc, ks, vc, vcs, Hq, Hkv, scale, rows, allowance, hw_err, jitter, jitter_seed,
                    t_shift=None):
    B, _, S, D = qc.shape
    r, n = _rows_arg(rows, S)
    o, lse = _out(B, Hq, n, D)
    al, ac, ap = ((np.empty_like(o) for _ in range(3)) if allowance else (None, None, None))
    le = np.empty_like(lse) if allowance else None
    args = [np.ascontiguousarray(a) for a in (qc, qs, kc, ks, vc, vcs)]
    extra = [] if t_shift is None else [int(t_shift)]
    fn(*[_ptr(a) for a in args], B, S, Hq, Hkv, D, float(scale), _ptr(r), n, *extra, _ptr(o), _ptr(lse),
       float(hw_err), _ptr(al), _ptr(ac), _ptr(ap), _ptr(le), float(jitter), int(jitter_seed))
    return (o, lse, Allowance(al, ac, ap, le)) if allowance else (o, lse)


def attn_completed(qc, qs, kc, ks, vc, vcs, Hq, Hkv, scale, rows=None, t_shift=0, allowance=False,
                   hw_err=HW_ERR, jitter=0.0, jitter_seed=0):
    """O7: completed-block partial (O_c [B,Hq,n,D], lse_c [B,Hq,n]) from codes in the ABI layouts.

    With ``allowance`` also returns the R15 Allowance (the largest change of O_c that a kernel on the
    block-scaled FP8 MFMA can make through the hardware's dot-product error and fp32 evaluation:
    (i) alternative valid P codes, (ii) the normaliser, (iii) P.V accumulation), for ``hw_err``
    times the measured error model (0 leaves fp32 evaluation only). ``jitter`` (test model of a
    kernel) moves each score by up to ``jitter`` times its bound."""
    return _completed_like(_load().orc_attn_completed, qc, qs, kc, ks, vc, vcs, Hq, Hkv, scale, rows, allowance,
                           hw_err, jitter, jitter_seed, t_shift=t_shift)


def attn_own(qc, qs, kc, ks, vt, vta, Hq, Hkv, scale, rows=None, allowance=False, hw_err=HW_ERR, jitter=0.0,
             jitter_seed=0):
    """O8: own-block partial (O_o, lse_o) on the token-normalised V. With ``allowance`` also the R15
    Allowance for a kernel whose own-block scores carry the hardware dot-product error (no code or
    P.V term: P is not quantised there)."""
    B, _, S, D = qc.shape
    r, n = _rows_arg(rows, S)
    o, lse = _out(B, Hq, n, D)
    al = np.empty_like(o) if allowance else None
    le = np.empty_like(lse) if allowance else None
    args = [np.ascontiguousarray(a) for a in (qc, qs, kc, ks, vt, vta)]
    _load().orc_attn_own(*[_ptr(a) for a in args], B, S, Hq, Hkv, D, float(scale), _ptr(r), n, _ptr(o), _ptr(lse),
                         float(hw_err), _ptr(al), _ptr(le), float(jitter), int(jitter_seed))
    if not allowance:
        return o, lse
    return o, lse, Allowance(al, np.zeros_like(al), np.zeros_like(al), le)


def attn_leaky(qc, qs, kc, ks, vc, vcs, Hq, Hkv, scale, rows=None, allowance=False, hw_err=HW_ERR, jitter=0.0,
               jitter_seed=0):
    """Ordinary causal MXFP8 (keys j <= i through the completed-block machinery, the last P block
    partial). ``allowance``, ``hw_err``, ``jitter``: as for attn_completed."""
    return _completed_like(_load().orc_attn_leaky, qc, qs, kc, ks, vc, vcs, Hq, Hkv, scale, rows, allowance, hw_err,
                           jitter, jitter_seed)


def lse_merge(oc, lsec, oo, lseo):
    """O9: merge two partials through their log-sum-exps."""
    oc, lsec, oo, lseo = (np.ascontiguousarray(a, dtype=np.float64) for a in (oc, lsec, oo, lseo))
    D = oc.shape[-1]
    n = lsec.size
    o = np.empty_like(oc)
    lse = np.empty_like(lsec)
    _load().orc_lse_merge(_ptr(oc), _ptr(lsec), _ptr(oo), _ptr(lseo), n, D, _ptr(o), _ptr(lse))
    return o, lse


def _raw3(fn, q, k, v, scale, rows):
    q, k, v = _as_view(q), _as_view(k), _as_view(v)
    r, n = _rows_arg(rows, q.S)
    o, lse = _out(q.B, q.H, n, q.D)
    fn(_ptr(q.data), q.sb, q.ss, q.sh, _ptr(k.data), k.sb, k.ss, k.sh, _ptr(v.data), v.sb, v.ss, v.sh,
       q.B, q.S, q.H, k.H, q.D, float(scale), _ptr(r), n, _ptr(o), _ptr(lse))
    return o, lse


def attn_reference(q, k, v, scale, rows=None):
    """Unquantised textbook causal attention in fp64 on the bf16 values."""
    return _raw3(_load().orc_attn_reference, q, k, v, scale, rows)


def attn_identity(q, k, v, scale, rows=None):
    """The split-and-merge structure with every quantiser replaced by the identity."""
    return _raw3(_load().orc_attn_identity, q, k, v, scale, rows)


@dataclass
class Quantized:
    qc: np.ndarray
    qs: np.ndarray
    kc: np.ndarray
    ks: np.ndarray
    vc: np.ndarray
    vcs: np.ndarray
    vt: np.ndarray
    vta: np.ndarray


def quantize_all(q, k, v) -> Quantized:
    qc, qs = quantize_rowwise(q)
    kc, ks = quantize_rowwise(k)
    vc, vcs, vt, vta = quantize_v(v)
    return Quantized(qc, qs, kc, ks, vc, vcs, vt, vta)


def forward(q, k, v, scale, rows=None, quant: Quantized | None = None, hw_err=HW_ERR):
    """The leak-free forward: quantise, completed partial, own partial, merge. Returns
    (O [B,Hq,n,D], lse [B,Hq,n], parts) where parts holds the partials, the quantised operands,
    "allowance": the R15 allowance of the merged output, i.e. each partial's allowance times its
    merge weight w = e^(lse_part - lse), plus the first-order effect of the partials' lse errors on
    the weights, w_c w_o |O_c - O_o| (err_c + err_o); "allowance_code" and "allowance_pv", its terms
    (i) (the alternative valid P codes of the completed partial) and (iii) (the P.V products the MFMA
    cuts), times w_c."""
    qv, kv = _as_view(q), _as_view(k)
    Hq, Hkv = qv.H, kv.H
    z = quant if quant is not None else quantize_all(q, k, v)
    oc, lc, ac = attn_completed(z.qc, z.qs, z.kc, z.ks, z.vc, z.vcs, Hq, Hkv, scale, rows, allowance=True,
                                hw_err=hw_err)
    oo, lo, ao = attn_own(z.qc, z.qs, z.kc, z.ks, z.vt, z.vta, Hq, Hkv, scale, rows, allowance=True, hw_err=hw_err)
    o, lse = lse_merge(oc, lc, oo, lo)
    with np.errstate(invalid="ignore"):
        wc = np.where(np.isneginf(lc), 0.0, np.exp(lc - lse))
    wo = np.exp(lo - lse)
    ec, eo = ac.lse_err, ao.lse_err
    al = wc[..., None] * ac.total + wo[..., None] * ao.total + (wc * wo * (ec + eo))[..., None] * np.abs(oc - oo)
    return o, lse, {"o_c": oc, "lse_c": lc, "o_o": oo, "lse_o": lo, "quant": z, "allowance_c": ac.total,
                    "allowance_o": ao.total, "allowance": al, "allowance_code": wc[..., None] * ac.code,
                    "allowance_pv": wc[..., None] * ac.pv, "lse_err": wc * ec + wo * eo}


def forward_leaky(q, k, v, scale, rows=None, quant: Quantized | None = None, allowance=False):
    """Ordinary causal MXFP8 forward (the variant that leaks through V scales); with ``allowance``
    also the R15 allowance and lse error bound, as attn_leaky."""
    qv, kv = _as_view(q), _as_view(k)
    z = quant if quant is not None else quantize_all(q, k, v)
    return attn_leaky(z.qc, z.qs, z.kc, z.ks, z.vc, z.vcs, qv.H, kv.H, scale, rows, allowance=allowance)


def attn_bwd_values(Q, K, V, O, dO, lse, scale, qrows=None, krows=None, allowance=False):
    """Backward of causal softmax attention at real-valued operands (Q, O, dO [B,Hq,S,D]; K, V
    [B,Hkv,S,D]; lse [B,Hq,S] natural log): (dq [B,Hq,nq,D], dk, dv [B,Hkv,nk,D]) for the query rows
    ``qrows`` and key rows ``krows`` (None: all rows). With ``allowance`` also (aq, ak, av): reading
    R16, the per-element bound of the bf16 rounding of P and dS as product operands."""
    arrs = [np.ascontiguousarray(a, dtype=np.float64) for a in (Q, K, V, O, dO, lse)]
    B, Hq, S, D = arrs[0].shape
    Hkv = arrs[1].shape[1]
    qr, nq = _rows_arg(qrows, S)
    kr, nk = _rows_arg(krows, S)
    dq = np.empty((B, Hq, nq, D))
    dk = np.empty((B, Hkv, nk, D))
    dv = np.empty((B, Hkv, nk, D))
    al = [np.empty_like(x) for x in (dq, dk, dv)] if allowance else [None, None, None]
    _load().orc_attn_bwd_values(*[_ptr(a) for a in arrs], B, S, Hq, Hkv, D, float(scale), _ptr(qr), nq, _ptr(kr), nk,
                                _ptr(dq), _ptr(dk), _ptr(dv), *[_ptr(a) for a in al])
    return (dq, dk, dv, *al) if allowance else (dq, dk, dv)


def attn_bwd(qc, qs, kc, ks, vt, vta, o, lse, do, scale, qrows=None, krows=None, allowance=False):
    """Backward on decoded operands from the codes (Q/K rowwise [B,H,S,D] + scales, V token-normalised
    [B,Hkv,S,D] + amplitudes [B,Hkv,S]), the forward's O (bf16 view), lse (fp32 [B,Hq,S]) and the
    output gradient dO (bf16 view): (dq [B,Hq,nq,D], dk, dv [B,Hkv,nk,D]) in fp64, and with
    ``allowance`` the R16 bounds (aq, ak, av) as attn_bwd_values."""
    ov, gv = _as_view(o), _as_view(do)
    B, Hq, S, D = qc.shape
    Hkv = kc.shape[1]
    qr, nq = _rows_arg(qrows, S)
    kr, nk = _rows_arg(krows, S)
    dq = np.empty((B, Hq, nq, D))
    dk = np.empty((B, Hkv, nk, D))
    dv = np.empty((B, Hkv, nk, D))
    al = [np.empty_like(x) for x in (dq, dk, dv)] if allowance else [None, None, None]
    args = [np.ascontiguousarray(a) for a in (qc, qs, kc, ks, vt, vta)]
    l32 = np.ascontiguousarray(lse, dtype=np.float32)
    _load().orc_attn_bwd(*[_ptr(a) for a in args], _ptr(ov.data), ov.sb, ov.ss, ov.sh, _ptr(l32), _ptr(gv.data), gv.sb,
                         gv.ss, gv.sh, B, S, Hq, Hkv, D, float(scale), _ptr(qr), nq, _ptr(kr), nk, _ptr(dq), _ptr(dk),
                         _ptr(dv), *[_ptr(a) for a in al])
    return (dq, dk, dv, *al) if allowance else (dq, dk, dv)
