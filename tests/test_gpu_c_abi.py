"""The C ABI from plain C: tests/c_abi/forward_from_c.c, built with gcc against include/mxfa.h,
libmxfa.so and the oracle library, quantises seeded inputs, runs the whole forward and checks it
(encoders bit-exact against the oracle's, mxfa_attn_fwd bit-exact against the chain of separate
entry points; at S = 32 the own-block entry point within 1e-4 * RMS of the oracle and the whole
forward within 2e-2 * RMS); no Python between the caller and the library."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_forward_from_c(tmp_path):
    lib_dir = os.path.join(ROOT, "causal_mxfp8_block_amd")
    orc_dir = os.path.join(ROOT, "oracle")
    for f in (os.path.join(lib_dir, "libmxfa.so"), os.path.join(orc_dir, "liboracle.so")):
        if not os.path.exists(f):
            raise RuntimeError(f"{f} is missing: build with __graft_entry__.build()")
    exe = str(tmp_path / "forward_from_c")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", orc_dir, "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi", "forward_from_c.c"),
           "-L", lib_dir, "-lmxfa", "-L", orc_dir, "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{lib_dir}:{orc_dir}:{os.path.join(ROCM, 'lib')}", "-o", exe]
    subprocess.run(cmd, check=True, timeout=120)
    print("running the C consumer (S = 32, 96)", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    assert r.returncode == 0 and "ALL OK" in r.stdout
