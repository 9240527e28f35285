"""Host-side checks of the C ABI (no GPU needed): libmxfa.so loads, exports every entry point that
include/mxfa.h declares, and rejects invalid arguments before touching a device."""
import ctypes
import os
import re

import pytest

import causal_mxfp8_block_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["mxfa_mxfp8_quantize", "mxfa_mxfp8_quantize_kv", "mxfa_attn_fwd_completed_blocks", "mxfa_attn_fwd_own_block",
              "mxfa_lse_merge", "mxfa_attn_fwd", "mxfa_attn_fwd_fused", "mxfa_attn_fwd_leaky",
              "mxfa_attn_fwd_workspace_bytes",
              "mxfa_status_string",
              "mxfa_last_error"]:
        assert n in names


def test_header_compiles_as_c_and_a_c_consumer_links(tmp_path):
    """include/mxfa.h is plain C (C99, warnings as errors), and the C consumer of the GPU tests
    (tests/c_abi/forward_from_c.c) links against libmxfa.so; the GPU test runs it."""
    import subprocess
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib_dir, orc_dir = os.path.dirname(mx.LIB_PATH), os.path.join(ROOT, "oracle")
    src = tmp_path / "h.c"
    src.write_text('#include "mxfa.h"\nint main(void) { return mxfa_status_string(MXFA_OK) == 0; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    "-c", str(src), "-o", str(tmp_path / "h.o")], check=True, timeout=60)
    if not os.path.exists(os.path.join(orc_dir, "liboracle.so")):
        pytest.skip("oracle library not built")
    subprocess.run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", orc_dir, "-I", os.path.join(rocm, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "forward_from_c.c"), "-L", lib_dir, "-lmxfa", "-L", orc_dir,
                    "-loracle", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm", "-o", str(tmp_path / "ffc")],
                   check=True, timeout=120)


def test_library_exports_every_declared_symbol():
    lib = mx.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_exports_nothing_undeclared():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", mx.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l and l.split()[-1].startswith("mxfa")}
    assert exported == set(declared_functions())


def _err(status):
    return status, mx.lib().mxfa_last_error().decode()


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced: validation fails first


@pytest.mark.parametrize("args,status,needle", [
    (dict(D=64), 3, "D = 64"),
    (dict(S=48), 2, "multiple of 32"),
    (dict(Hq=6, Hkv=4), 2, "multiple of Hkv"),
    (dict(B=0), 2, ">= 1"),
    (dict(qc=None), 1, "qc is NULL"),
    (dict(vcs=FAKE + 4), 4, "vcs is not 16-byte aligned"),
])
def test_completed_validation(args, status, needle):
    a = dict(qc=FAKE, qs=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vcs=FAKE, B=1, S=64, Hq=4, Hkv=2, D=128)
    a.update(args)
    st, msg = _err(mx.lib().mxfa_attn_fwd_completed_blocks(a["qc"], a["qs"], a["kc"], a["ks"], a["vc"], a["vcs"],
                                                           a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], 0.1, FAKE,
                                                           FAKE, None))
    assert st == status and needle in msg, (st, msg)


def test_quantize_validation():
    L = mx.lib()
    st, msg = _err(L.mxfa_mxfp8_quantize(FAKE, 1, 64, 2, 128, 64 * 256, 256, 128, 7, FAKE, FAKE, None, None, None))
    assert st == 3 and "mode" in msg
    st, msg = _err(L.mxfa_mxfp8_quantize(FAKE, 1, 64, 2, 128, 64 * 256, 256, 12, 0, FAKE, FAKE, None, None, None))
    assert st in (2, 4)
    st, msg = _err(L.mxfa_mxfp8_quantize(FAKE, 1, 64, 2, 128, 64 * 256, 256, 128, 0, FAKE, FAKE, FAKE, FAKE, None))
    assert st == 3 and "token-normalised" in msg
    st, msg = _err(L.mxfa_mxfp8_quantize(FAKE, 1, 40, 2, 128, 40 * 256, 256, 128, 1, FAKE, FAKE, None, None, None))
    assert st == 2


def test_quantize_kv_validation():
    L = mx.lib()
    ok = (FAKE, 64 * 256, 256, 128)
    st, msg = _err(L.mxfa_mxfp8_quantize_kv(*ok, *ok, 1, 64, 2, 64, *[FAKE] * 6, None))
    assert st == 3 and "D = 64" in msg
    st, msg = _err(L.mxfa_mxfp8_quantize_kv(*ok, *ok, 1, 40, 2, 128, *[FAKE] * 6, None))
    assert st == 2 and "multiple of 32" in msg
    st, msg = _err(L.mxfa_mxfp8_quantize_kv(*ok, *ok, 1, (1 << 24) + 32, 2, 128, *[FAKE] * 6, None))
    assert st == 2 and "2^24" in msg
    st, msg = _err(L.mxfa_mxfp8_quantize_kv(*ok, FAKE, 64 * 256, 256, 12, 1, 64, 2, 128, *[FAKE] * 6, None))
    assert st in (2, 4)
    st, msg = _err(L.mxfa_mxfp8_quantize_kv(*ok, *ok, 1, 64, 2, 128, *[FAKE] * 5, None, None))
    assert st == 1 and "v_tn_amps" in msg


def test_merge_and_forward_validation():
    L = mx.lib()
    st, msg = _err(L.mxfa_lse_merge(FAKE, FAKE, FAKE, FAKE, 1, 64, 2, 128, FAKE, 64 * 256, 256, 128, 5, None, None))
    assert st == 3
    need = L.mxfa_attn_fwd_workspace_bytes(1, 64, 4, 2, 128)
    assert need > 0
    st, msg = _err(L.mxfa_attn_fwd(FAKE, 64 * 512, 512, 128, FAKE, 64 * 256, 256, 128, FAKE, 64 * 256, 256, 128,
                                   1, 64, 4, 2, 128, 0.1, FAKE, need - 1, FAKE, 64 * 512, 512, 128, 0, None, None))
    assert st == 3 and "workspace" in msg
    st, msg = _err(L.mxfa_attn_fwd(FAKE, 64 * 512, 512, 128, FAKE, 64 * 256, 256, 128, FAKE, 64 * 256, 256, 128,
                                   1, 64, 4, 2, 128, 0.1, FAKE + 256 * 3 + 16, need, FAKE, 64 * 512, 512, 128, 0,
                                   None, None))
    assert st == 4


def test_no_device_is_an_error_not_a_crash():
    """Valid arguments on a machine without a gfx950 device return MXFA_ERR_NO_DEVICE."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, msg = _err(mx.lib().mxfa_attn_fwd_completed_blocks(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 4, 2, 128,
                                                           0.1, FAKE, FAKE, None))
    assert st == 5, msg


@pytest.mark.parametrize("args,status,needle", [
    (dict(D=96), 3, "D = 96"),
    (dict(S=40), 2, "multiple of 32"),
    (dict(vc=None), 1, "vc is NULL"),
    (dict(dtype=5), 3, "output dtype"),
    (dict(osh=100), 4, "multiples of 8"),
])
def test_leaky_validation(args, status, needle):
    a = dict(qc=FAKE, qs=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vcs=FAKE, B=1, S=64, Hq=4, Hkv=2, D=128, osh=128,
             dtype=0)
    a.update(args)
    S, Hq = a["S"], a["Hq"]
    st, msg = _err(mx.lib().mxfa_attn_fwd_leaky(a["qc"], a["qs"], a["kc"], a["ks"], a["vc"], a["vcs"], a["B"], S, Hq,
                                                a["Hkv"], a["D"], 0.1, FAKE, S * Hq * 128, Hq * 128, a["osh"],
                                                a["dtype"], None, None))
    assert st == status and needle in msg, (st, msg)


@pytest.mark.parametrize("args,status,needle", [
    (dict(D=64), 3, "D = 64"),
    (dict(S=80), 2, "multiple of 32"),
    (dict(Hq=3, Hkv=2), 2, "multiple of Hkv"),
    (dict(lse=None), 1, "lse is NULL"),
    (dict(dout=FAKE + 8), 4, "dout is not 16-byte aligned"),
    (dict(ksh=100), 4, "multiples of 8"),
    (dict(qss=64), 2, "overlap"),
    (dict(ws=None), 1, "workspace is NULL"),
    (dict(ws=FAKE + 16), 4, "256-byte aligned"),
    (dict(ws_short=True), 3, "workspace"),
])
def test_backward_validation(args, status, needle):
    """mxfa_attn_bwd refuses bad shapes, pointers, views and workspaces before any device work."""
    a = dict(B=1, S=64, Hq=4, Hkv=2, D=128, lse=FAKE, dout=FAKE, ws=FAKE, ws_short=False, ksh=128, qss=512)
    a.update(args)
    L = mx.lib()
    S, Hq, Hkv = a["S"], a["Hq"], a["Hkv"]
    need = L.mxfa_attn_bwd_workspace_bytes(a["B"], S, Hq, Hkv, 128) if a["D"] == 128 else 1 << 20
    assert need > 0
    st, msg = _err(L.mxfa_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["lse"], a["dout"], a["B"], S, Hq, Hkv,
                                   a["D"], 0.1, S * Hq * 128, a["qss"], 128, S * Hkv * 128, Hkv * 128, a["ksh"],
                                   a["ws"], need - 1 if a["ws_short"] else need, FAKE, FAKE, FAKE, None))
    assert st == status and needle in msg, (st, msg)


def test_backward_workspace_grows_with_the_problem():
    L = mx.lib()
    small = L.mxfa_attn_bwd_workspace_bytes(1, 64, 4, 2, 128)
    assert small > 0
    assert L.mxfa_attn_bwd_workspace_bytes(1, 128, 4, 2, 128) > small
    assert L.mxfa_attn_bwd_workspace_bytes(2, 64, 4, 2, 128) > small


@pytest.mark.parametrize("args,status,needle", [
    (dict(D=32), 3, "D = 32"),
    (dict(vt=None), 1, "vt is NULL"),
    (dict(oss=136), 4, "multiples of 16"),
    (dict(o=FAKE + 4), 4, "o_codes is not 16-byte aligned"),
    (dict(lse=FAKE + 4), 4, "lse_out is not 16-byte aligned"),
])
def test_fused_mxfp8_validation(args, status, needle):
    """The MXFP8-output forward needs 16-element strides (16-byte code rows) and checks them first."""
    a = dict(D=128, vt=FAKE, oss=4 * 128, o=FAKE, lse=FAKE)
    a.update(args)
    S, Hq = 64, 4
    st, msg = _err(mx.lib().mxfa_attn_fwd_fused_mxfp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["vt"], FAKE, 1, S, Hq, 2,
                                                      a["D"], 0.1, a["o"], S * Hq * 128, a["oss"], 128, FAKE,
                                                      a["lse"], None))
    assert st == status and needle in msg, (st, msg)


@pytest.mark.parametrize("args,status,needle", [
    (dict(D=64), 3, "D = 64"),
    (dict(q=None), 1, "q is NULL"),
    (dict(qsh=12), 4, "multiples of 8"),
    (dict(vt=None), 1, "vt is NULL"),
    (dict(dtype=3), 3, "output dtype"),
])
def test_fused_bf16q_validation(args, status, needle):
    a = dict(D=128, q=FAKE, qsh=128, vt=FAKE, dtype=0)
    a.update(args)
    S, Hq = 64, 4
    st, msg = _err(mx.lib().mxfa_attn_fwd_fused_bf16q(a["q"], S * Hq * 128, Hq * 128, a["qsh"], FAKE, FAKE, FAKE, FAKE,
                                                      a["vt"], FAKE, 1, S, Hq, 2, a["D"], 0.1, FAKE, S * Hq * 128,
                                                      Hq * 128, 128, a["dtype"], None, None))
    assert st == status and needle in msg, (st, msg)


BIG_S = (1 << 24) + 32  # the first multiple of 32 above the largest supported length


def test_sequence_length_bound_is_enforced():
    """S > 2^24 is refused by every entry point that takes S, before any device work (the kernels
    address a (b, head) slice of S * 128 code bytes with 32-bit offsets)."""
    L = mx.lib()
    S = BIG_S
    st, msg = _err(L.mxfa_attn_fwd_completed_blocks(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, S, 4, 2, 128, 0.1, FAKE,
                                                    FAKE, None))
    assert st == 2 and "2^24" in msg, (st, msg)
    st, msg = _err(L.mxfa_attn_fwd_own_block(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, S, 4, 2, 128, 0.1, FAKE, FAKE,
                                             None))
    assert st == 2 and "2^24" in msg, (st, msg)
    st, msg = _err(L.mxfa_attn_fwd_fused_bf16q(FAKE, S * 512, 512, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, S, 4,
                                               2, 128, 0.1, FAKE, S * 512, 512, 128, 0, None, None))
    assert st == 2 and "2^24" in msg, (st, msg)
    st, msg = _err(L.mxfa_attn_fwd_leaky(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, S, 4, 2, 128, 0.1, FAKE, S * 512, 512,
                                         128, 0, None, None))
    assert st == 2 and "2^24" in msg, (st, msg)
    for mode in (0, 1):
        st, msg = _err(L.mxfa_mxfp8_quantize(FAKE, 1, S, 2, 128, S * 256, 256, 128, mode, FAKE, FAKE,
                                             FAKE if mode else None, FAKE if mode else None, None))
        assert st == 2 and "2^24" in msg, (st, msg)
    st, msg = _err(L.mxfa_lse_merge(FAKE, FAKE, FAKE, FAKE, 1, S, 2, 128, FAKE, S * 256, 256, 128, 0, None, None))
    assert st == 2 and "2^24" in msg, (st, msg)
    assert L.mxfa_attn_fwd_workspace_bytes(1, S, 4, 2, 128) == 0
    assert L.mxfa_attn_bwd_workspace_bytes(1, S, 4, 2, 128) == 0
    # the largest supported length itself passes the shape checks (and stops at the device check here)
    st, msg = _err(L.mxfa_attn_fwd_completed_blocks(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1 << 24, 4, 2, 128, 0.1,
                                                    FAKE, FAKE, None))
    assert st != 2, msg


def test_noalloc_refuses_oversized_problems_before_device_work():
    """mxfa_attn_fwd_noalloc checks the problem against its static workspace on the host: a problem
    needing more than MXFA_NOALLOC_WORKSPACE_BYTES of K/V encodings is refused, naming the limit."""
    L = mx.lib()
    S, Hkv = 65536, 16
    assert L.mxfa_attn_fwd_workspace_bytes(1, S, 16, Hkv, 128) > mx.NOALLOC_WORKSPACE_BYTES
    st, msg = _err(L.mxfa_attn_fwd_noalloc(FAKE, S * 2048, 2048, 128, FAKE, S * 2048, 2048, 128, FAKE, S * 2048, 2048,
                                           128, 1, S, 16, Hkv, 128, 0.1, FAKE, S * 2048, 2048, 128, 0, None, None))
    assert st == 3 and "static workspace" in msg, (st, msg)
    with open(HEADER) as f:
        assert f"MXFA_NOALLOC_WORKSPACE_BYTES ((size_t)256 << 20)" in f.read()
    assert mx.NOALLOC_WORKSPACE_BYTES == 256 << 20
