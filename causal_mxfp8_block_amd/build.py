"""Build libmxfa.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmxfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
    # packed fp32 ops stay off: scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source extra flags. The backward kernels run one or two waves per SIMD, so their LDS operand reads
# must be issued well ahead of the MFMAs that use them: the ILP-first machine scheduler does that, the
# default occupancy-first one sinks each read next to its use.
EXTRA = {"attn_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))) + [os.path.join(PKG, "csrc", "api.cpp")]


def _clean(stderr: str) -> str:
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in (stderr or "").splitlines() if noise not in l)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 into causal_mxfp8_block_amd/libmxfa.so (always rebuilds)."""
    tag = f".tmp{os.getpid()}"
    inc = ["-I", os.path.join(ROOT, "include")]
    objs, procs = [], []
    for src in sources():  # one object per source (own flags), compiled in parallel, then one link
        obj = os.path.join(PKG, "csrc", os.path.basename(src) + tag + ".o")
        cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), *inc, "-c", "-o", obj, src]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    errs = []
    try:
        for src, pr in procs:
            _, stderr = pr.communicate()
            err = _clean(stderr)
            if pr.returncode != 0:
                errs.append(f"{os.path.basename(src)}: hipcc failed ({pr.returncode}):\n{err}")
            elif verbose and err.strip():
                print(err)
        if errs:
            raise RuntimeError("\n".join(errs))
        tmp = LIB + tag
        res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_clean(res.stderr)}")
        os.replace(tmp, LIB)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB


PEAK_SRC = os.path.join(PKG, "peak", "mfma_peak.hip")
PEAK_LIB = os.path.join(PKG, "libmxfa_peak.so")


def build_peak() -> str:
    """Compile the benchmark's MFMA throughput probe into causal_mxfp8_block_amd/libmxfa_peak.so."""
    tmp = PEAK_LIB + f".tmp{os.getpid()}"
    res = subprocess.run([HIPCC, *FLAGS, "-shared", "-o", tmp, PEAK_SRC], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"mfma_peak build failed ({res.returncode}):\n{_clean(res.stderr)}")
    os.replace(tmp, PEAK_LIB)
    return PEAK_LIB


if __name__ == "__main__":
    print(build(verbose=True))
