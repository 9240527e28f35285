"""Build and call the test-only hardware probes in hw_probe.hip (scaled FP8 MFMA scores, fp32 -> E4M3
conversion). Test infrastructure: nothing in the library imports this."""
from __future__ import annotations

import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hw_probe.hip")
LIB_PATH = os.path.join(_HERE, "libhw_probe.so")
_lib = None


def build() -> str:
    """Compile libhw_probe.so for gfx950 (always rebuilds)."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", tmp, _SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hw_probe build failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.probe_scores.argtypes = [P, P, P, P, I, I, P]
        L.probe_scores.restype = I
        L.probe_cvt.argtypes = [P, I, P]
        L.probe_cvt.restype = I
        _lib = L
    return _lib


def scores(kc, ks, qc, qs):
    """fp32 scores [nq, nk] of torch uint8 device tensors kc [nk,128], ks [nk,4], qc [nq,128], qs [nq,4]."""
    import torch
    nk, nq = kc.shape[0], qc.shape[0]
    out = torch.empty((nq, nk), dtype=torch.float32, device=kc.device)
    st = lib().probe_scores(kc.data_ptr(), ks.data_ptr(), qc.data_ptr(), qs.data_ptr(), nk, nq, out.data_ptr())
    if st != 0:
        raise RuntimeError(f"probe_scores: HIP error {st}")
    return out


def cvt_e4m3(x):
    """E4M3 codes (uint8, same length) of a torch float32 device vector whose length is a multiple of 4."""
    import torch
    n = x.numel()
    out = torch.empty(n // 4, dtype=torch.int32, device=x.device)
    st = lib().probe_cvt(x.data_ptr(), n, out.data_ptr())
    if st != 0:
        raise RuntimeError(f"probe_cvt: HIP error {st}")
    return out.view(torch.uint8)
