"""Helpers for the GPU parity tests: move seeded inputs to the device, run the HIP path through the
C ABI binding, sample rows, and compare against the oracle with a report of the worst elements."""
from __future__ import annotations

import sys

import numpy as np
import torch

import causal_mxfp8_block_amd as mx
import oracle

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def oracle_view(inp, name):
    x = getattr(inp, name)
    return oracle.BF16View.sbhd(x) if inp.workload.layout == "sbhd" else oracle.BF16View.bshd(x)


def gpu_quantize(inp):
    lay = inp.workload.layout
    q, k, v = (to_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    qc, qs = mx.mxfp8_quantize(q, "rowwise", lay)
    kc, ks = mx.mxfp8_quantize(k, "rowwise", lay)
    vc, vcs, vt, vta = mx.mxfp8_quantize(v, "v", lay)
    return dict(qc=qc, qs=qs, kc=kc, ks=ks, vc=vc, vcs=vcs, vt=vt, vta=vta)


def gpu_forward(inp, out_dtype=torch.float32):
    """Whole forward through mxfa_attn_fwd; returns (O [B,Hq,S,D] float64 numpy, lse [B,Hq,S])."""
    lay = inp.workload.layout
    q, k, v = (to_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    out, lse = mx.attn_fwd(q, k, v, inp.workload.scale, layout=lay, out_dtype=out_dtype)
    torch.cuda.synchronize()
    o = out.float()
    o = o.permute(0, 2, 1, 3) if lay == "bshd" else o.permute(1, 2, 0, 3)
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def sample_rows(S: int, seed: int, n_random: int = 192, head: int = 96, tail: int = 32, stride: int = 1024):
    """Rows 0..head-1, every stride-th row, the last `tail` rows and n_random seeded uniform rows."""
    rng = np.random.default_rng(seed + 1000)
    rows = set(range(min(head, S))) | set(range(0, S, stride)) | set(range(max(0, S - tail), S))
    rows |= set(rng.integers(0, S, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int32)


def uniform_rows(S: int, seed: int, n: int = 256):
    rng = np.random.default_rng(seed + 2000)
    return np.unique(rng.integers(0, S, size=n)).astype(np.int32)


def report(name, got, ref, rms, rows=None, allowance=None, tol=None, k=5):
    """Prints the comparison and returns max(|err| - allowance) / rms (the gated figure).

    ``allowance`` (oracle reading R15) is the largest change that alternative valid P codes can
    make per element; without it the gated figure is max|err| / rms."""
    err = np.abs(got - ref)
    al = np.zeros_like(err) if allowance is None else allowance
    excess = err - al
    gated = excess.max() / rms
    msg = (f"[{name}] max|err|/rms = {err.max() / rms:.3e}  rms(err)/rms = {np.sqrt(np.mean(err ** 2)) / rms:.3e}"
           f"  rms(ref) = {rms:.3e}")
    if allowance is not None:
        msg += f"  max(|err|-allow)/rms = {gated:.3e}  mean(allow)/rms = {al.mean() / rms:.2e}"
        if tol is not None:
            msg += f"  elements over tol without allowance: {int(np.sum(err > tol * rms))} of {err.size}"
    say(msg)
    worst = np.argsort(excess.reshape(-1))[::-1][:k]
    for w in worst:
        idx = np.unravel_index(w, err.shape)
        row = rows[idx[2]] if rows is not None and len(idx) > 2 else (idx[2] if len(idx) > 2 else None)
        say(f"    at (b, h, row, d) = ({idx[0]}, {idx[1]}, {row}, {idx[-1] if len(idx) > 3 else '-'}): "
            f"got {got[idx]:.6e} ref {ref[idx]:.6e} allowance {al[idx]:.3e}")
    return gated


def gate(name, got, ref, rms, rows=None, allowance=None, allowance_hw=None, tol=2e-2, max_over_frac=None,
         max_rms_err=1e-2, k=5):
    """The forward parity gate, with what the R15 allowance absorbs made explicit. Asserts and prints.

    err = |got - ref|, plain tolerance tol * rms (the stated bound max|err| <= tol * RMS).
    ``allowance`` is the oracle's whole R15 allowance per element; ``allowance_hw`` its hardware
    terms: (i) the change alternative valid P codes of the completed blocks can make and (iii) the
    P.V products the block-scaled MFMA cuts (its measured arithmetic, pinned by the probe tests).
    The rest is the normaliser, own-block and merge-weight terms, of the size of the score error
    bound times |O|.
      (a) every element: err <= tol * rms + allowance;
      (b) every element with err > tol * rms has a nonzero hardware term, and its excess over the
          plain tolerance and the other terms lies within the hardware terms;
      (c) the fraction of elements with err > tol * rms is at most ``max_over_frac``;
      (d) rms(err) <= max_rms_err * rms.
    Prints the raw max|err| / rms, rms(err) / rms, the count over the plain tolerance and the
    largest share of the hardware terms such an element needs. Returns those figures."""
    err = np.abs(got - ref)
    al = np.zeros_like(err) if allowance is None else allowance
    hw = np.zeros_like(err) if allowance_hw is None else allowance_hw
    rest = al - hw
    plain = tol * rms
    over = err > plain
    n_over = int(over.sum())
    need = np.where(over & (hw > 0), (err - plain - rest) / np.where(hw > 0, hw, 1.0), 0.0)
    stats = dict(max_err=float(err.max() / rms), rms_err=float(np.sqrt(np.mean(err ** 2)) / rms), n_over=n_over,
                 n=int(err.size), frac_over=n_over / err.size, gated=float((err - al).max() / rms),
                 hw_share=float(need.max()) if n_over else 0.0)
    say(f"[{name}] max|err|/rms = {stats['max_err']:.3e}  rms(err)/rms = {stats['rms_err']:.3e}  "
        f"over {tol:g}*rms: {n_over} of {err.size} ({stats['frac_over']:.2e})  "
        f"max(|err|-allowance)/rms = {stats['gated']:.3e}  largest hardware-term share used = {stats['hw_share']:.3f}  "
        f"rms(ref) = {rms:.3e}")
    worst = np.argsort((err - al).reshape(-1))[::-1][:k]
    for w in worst:
        idx = np.unravel_index(w, err.shape)
        row = rows[idx[2]] if rows is not None and len(idx) > 2 else (idx[2] if len(idx) > 2 else None)
        say(f"    at (b, h, row, d) = ({idx[0]}, {idx[1]}, {row}, {idx[-1] if len(idx) > 3 else '-'}): "
            f"got {got[idx]:.6e} ref {ref[idx]:.6e} allowance {al[idx]:.3e} (hardware terms {hw[idx]:.3e})")
    assert (err - al).max() <= plain, f"{name}: an element exceeds the tolerance plus the allowance"
    assert np.all(hw[over] > 0), f"{name}: an element over the plain tolerance has no hardware term"
    assert np.all(need <= 1.0 + 1e-9), f"{name}: an excess over the plain tolerance exceeds the hardware terms"
    if max_over_frac is not None:
        assert stats["frac_over"] <= max_over_frac, f"{name}: {n_over} elements over the plain tolerance"
    assert stats["rms_err"] <= max_rms_err, f"{name}: rms(err) / rms = {stats['rms_err']:.3e}"
    return stats
