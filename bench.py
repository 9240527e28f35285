"""Benchmark: leak-free causal MXFP8 attention forward on one MI355X.

One step is one pass of the whole forward path over one batch: MXFP8 quantisation of Q, K (rowwise)
and V (columnwise + token-normalised; K and V in one launch), then the completed-block partial, the
own-block partial and the LSE merge (bf16 output) -- by default in one fused kernel that also
quantises Q (`--path fused`), or as three separate kernels after a separate Q quantiser
(`--path stepwise`) -- each call through the C ABI of libmxfa.so on torch's current stream.
`--path leaky` times ordinary causal MXFP8 instead (the variant the method replaces), for the
own-block/ordinary comparison the published timings make.
Inputs are seeded synthetic bf16 tensors already resident in HBM when the timed region starts.

Workload (the configuration the published forward timings are quoted on): B=1, 16 query heads,
4 KV heads, S=32768, D=128, BSHD, causal, V rows scaled by 2^e, e ~ U{-4..4} per (token, kv-head).

Prints one JSON line. `value` is TFLOP/s of the whole forward with the FlashAttention causal count
2*B*Hq*S^2*D; `roofline` is the attention kernel (the dominant one: fused, leaky, or completed-block
when stepwise) against the MXFP8 MFMA peak, from HIP events around its launches in the timed steps; `cpu_baseline` times the fp64 CPU
oracle on a bounded row sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal MXFP8 attn fwd TFLOP/s + ms at B=1,H=16/4,S=32K,D=128; % MFMA peak"
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8/MXFP8 MFMA
HBM_PEAK_GBS = 8000.0
# Published own-block forward times (B200, BSHD, batch 1, includes quantisation), ms, keyed by
# (Hq, Hkv, S): TransformerEngine PR #3865, "Performance". Context from other hardware, not a target;
# e.g. 2*1*16*32768^2*128 / 2.797 ms = 1572.4 TFLOP/s at the headline workload.
PAGES_OWN_BLOCK_MS = {(16, 4, 8192): 1.054, (16, 4, 16384): 1.075, (16, 4, 32768): 2.797,
                      (16, 16, 8192): 1.081, (16, 16, 16384): 1.077, (16, 16, 32768): 3.041}
# Published own-block forward+backward for B=1, 16/16 heads, S=32768 (B200): 12.799 ms; with the
# FlashAttention count (backward = 2.5 x forward) that is 3.5 * 2*16*32768^2*128 / 12.799 ms.
METRIC_FWDBWD = "causal MXFP8 attn fwd + bf16 bwd TFLOP/s + ms at B=1,H=16/16,S=32K,D=128 SBHD"
PAGES_FWDBWD_TFLOPS = 3.5 * 2 * 16 * 32768 ** 2 * 128 / 12.799e-3 / 1e12
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def completed_pairs(B, Hq, S):
    n = S // 32
    return B * Hq * 1024 * (n * (n - 1) // 2)  # sum_i 32*floor(i/32) over i < S


def own_pairs(B, Hq, S):
    return B * Hq * (S // 32) * (32 * 33 // 2)


def read_traffic(kernel_source: str, kernel: str):
    """HBM traffic of the attention kernel per launch from the committed PMC summary, or None when
    the summary is missing or was taken on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_kernel_gqa16x4_s32k_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = hashlib.sha256(open(kernel_source, "rb").read()).hexdigest()[:16]
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != sha:
        return None
    return float(t.group(1))


def cpu_baseline(inp, rows_n: int, seed: int = 0):
    """The oracle as it stands on a row sample of the same workload (quantisation of the whole
    tensors included); TFLOP/s counts 4*D per (query, visible key) pair of the sampled rows."""
    import oracle
    w = inp.workload
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(w.S, size=rows_n, replace=False)).astype(np.int32)
    view = oracle.BF16View.sbhd if w.layout == "sbhd" else oracle.BF16View.bshd
    q, k, v = view(inp.q), view(inp.k), view(inp.v)
    oracle.build()
    t0 = time.perf_counter()
    z = oracle.quantize_all(q, k, v)
    oc, lc = oracle.attn_completed(z.qc, z.qs, z.kc, z.ks, z.vc, z.vcs, w.Hq, w.Hkv, w.scale, rows)
    oo, lo = oracle.attn_own(z.qc, z.qs, z.kc, z.ks, z.vt, z.vta, w.Hq, w.Hkv, w.scale, rows)
    oracle.lse_merge(oc, lc, oo, lo)
    dt = time.perf_counter() - t0
    flops = float(np.sum(4.0 * w.D * (rows.astype(np.float64) + 1)) * w.B * w.Hq)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    cores = min(cores, os.cpu_count() or cores)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows_n} seeded random query rows x {w.Hq} heads of {w.name} (all keys of each row), "
                      f"plus quantisation of the whole Q/K/V; {dt:.1f} s wall"}


def measure_mfma_peak(torch, reps: int = 5):
    """Measured FP8 MFMA throughput of the device (TFLOP/s): the best of ``reps`` launches of the
    probe in libmxfa_peak.so (independent v_mfma_scale_f32_32x32x64_f8f6f4 chains, two or more waves
    per SIMD, nothing else), HIP events on torch's current stream."""
    import ctypes
    from causal_mxfp8_block_amd import build as b
    if not os.path.exists(b.PEAK_LIB):
        b.build_peak()
    L = ctypes.CDLL(b.PEAK_LIB)
    L.mxfa_peak_mfma_fp8.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.mxfa_peak_mfma_fp8.restype = ctypes.c_int
    blocks, iters = 1024, 64
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    flop = blocks * 8 * 4 * iters * (32 * 32 * 64 * 2)
    best = None
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = L.mxfa_peak_mfma_fp8(blocks, iters, out.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        if st != 0:
            raise RuntimeError(f"mfma peak probe: HIP error {st}")
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        if r > 0:  # the first launch loads the module
            best = ms if best is None else min(best, ms)
    return flop / (best * 1e-3) / 1e12


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa16x4_s32k_amplitudes")
    ap.add_argument("--path", choices=["fused", "stepwise", "leaky", "mxfp8_out"], default="fused",
                    help="fused (default): the leak-free forward in one attention kernel; stepwise: its three "
                         "separate kernels; leaky: ordinary causal MXFP8 (the variant the method replaces); "
                         "mxfp8_out: the fused kernel with its output in MXFP8 (E4M3 codes + E8M0 per 32 columns)")
    ap.add_argument("--cpu-rows", type=int, default=8192, help="rows of the oracle CPU-baseline sample (0 skips)")
    ap.add_argument("--mode", choices=["fwd", "fwdbwd", "peak"], default="fwd",
                    help="fwd (default): the forward metric; fwdbwd: forward + bf16 backward on decoded operands "
                         "(default workload mha16_s32k_sbhd, the configuration the published fwd+bwd times use); "
                         "peak: only the measured FP8 MFMA throughput of the device")
    ap.add_argument("--copy-only", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times): the calibration for HBM counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_only:
        n = args.copy_only << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n}), flush=True)
        return
    import causal_mxfp8_block_amd as mx
    from causal_mxfp8_block_amd.inputs import WORKLOADS, make_inputs

    if args.mode == "peak":
        tf = measure_mfma_peak(torch)
        print(json.dumps({"metric": "measured FP8 MFMA throughput (v_mfma_scale_f32_32x32x64_f8f6f4)",
                          "value": round(tf, 1), "unit": "TFLOP/s", "nominal": MFMA_FP8_PEAK_TFLOPS,
                          "frac_of_nominal": round(tf / MFMA_FP8_PEAK_TFLOPS, 4)}), flush=True)
        return
    if args.mode == "fwdbwd":
        return run_fwdbwd(args, torch, mx, WORKLOADS, make_inputs)
    w = WORKLOADS[args.workload]
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = to(inp.q), to(inp.k), to(inp.v)
    lay = w.layout
    B, S, Hq, Hkv, D = w.B, w.S, w.Hq, w.Hkv, w.D
    u8, f32 = dict(dtype=torch.uint8, device=dev), dict(dtype=torch.float32, device=dev)
    qc, qs = torch.empty((B, Hq, S, D), **u8), torch.empty((B, Hq, S, D // 32), **u8)
    kc, ks = torch.empty((B, Hkv, S, D), **u8), torch.empty((B, Hkv, S, D // 32), **u8)
    vc, vcs = torch.empty((B, Hkv, D, S), **u8), torch.empty((B, Hkv, S // 32, D), **u8)
    vt, vta = torch.empty((B, Hkv, S, D), **u8), torch.empty((B, Hkv, S), **u8)
    stepwise_buffers = args.path == "stepwise"
    oc, lc = (torch.empty((B, Hq, S, D), **f32), torch.empty((B, Hq, S), **f32)) if stepwise_buffers else (None, None)
    oo, lo = (torch.empty((B, Hq, S, D), **f32), torch.empty((B, Hq, S), **f32)) if stepwise_buffers else (None, None)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    mx8 = args.path == "mxfp8_out"
    out8 = torch.empty(q.shape, **u8) if mx8 else None  # E4M3 codes in O's layout
    sf_o = torch.empty((B, Hq, S, D // 32), **u8) if mx8 else None
    lse = torch.empty((B, Hq, S), **f32)
    L = mx.lib()
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    fused = args.path == "fused"
    leaky = args.path == "leaky"
    # The fused path quantises Q inside the attention kernel (attn_fwd_fused_bf16q, what attn_fwd runs);
    # the stepwise and leaky paths take Q's codes from the rowwise quantiser.
    names = (["quantize_kv", "fused"] if fused else
             ["quantize_q", "quantize_kv"] + (["leaky"] if leaky else ["fused_mxfp8"] if mx8 else
                                                           ["completed", "own_block", "merge"]))

    def view(t):
        return mx.view_of(t, lay)

    qv, kv_, vv, ov = view(q), view(k), view(v), view(out)
    ov8 = view(out8) if mx8 else None

    def step(evs=None):
        calls = [] if fused else [
            lambda: L.mxfa_mxfp8_quantize(q.data_ptr(), B, S, Hq, D, *qv[4:], mx.ROWWISE, qc.data_ptr(),
                                          qs.data_ptr(), None, None, sh)]
        # K and V in one launch, as attn_fwd encodes them
        calls.append(lambda: L.mxfa_mxfp8_quantize_kv(k.data_ptr(), *kv_[4:], v.data_ptr(), *vv[4:], B, S, Hkv, D,
                                                      kc.data_ptr(), ks.data_ptr(), vc.data_ptr(), vcs.data_ptr(),
                                                      vt.data_ptr(), vta.data_ptr(), sh))
        if leaky:
            calls.append(lambda: L.mxfa_attn_fwd_leaky(qc.data_ptr(), qs.data_ptr(), kc.data_ptr(), ks.data_ptr(),
                                                       vc.data_ptr(), vcs.data_ptr(), B, S, Hq, Hkv, D, w.scale,
                                                       out.data_ptr(), *ov[4:], mx.OUT_BF16, lse.data_ptr(), sh))
        elif mx8:
            calls.append(lambda: L.mxfa_attn_fwd_fused_mxfp8(qc.data_ptr(), qs.data_ptr(), kc.data_ptr(), ks.data_ptr(),
                                                             vc.data_ptr(), vcs.data_ptr(), vt.data_ptr(),
                                                             vta.data_ptr(), B, S, Hq, Hkv, D, w.scale,
                                                             out8.data_ptr(), *ov8[4:], sf_o.data_ptr(),
                                                             lse.data_ptr(), sh))
        elif fused:
            calls.append(lambda: L.mxfa_attn_fwd_fused_bf16q(q.data_ptr(), *qv[4:], kc.data_ptr(), ks.data_ptr(),
                                                             vc.data_ptr(), vcs.data_ptr(), vt.data_ptr(),
                                                             vta.data_ptr(), B, S, Hq, Hkv, D, w.scale, out.data_ptr(),
                                                             *ov[4:], mx.OUT_BF16, lse.data_ptr(), sh))
        else:
            calls += [
                lambda: L.mxfa_attn_fwd_completed_blocks(qc.data_ptr(), qs.data_ptr(), kc.data_ptr(), ks.data_ptr(),
                                                         vc.data_ptr(), vcs.data_ptr(), B, S, Hq, Hkv, D, w.scale,
                                                         oc.data_ptr(), lc.data_ptr(), sh),
                lambda: L.mxfa_attn_fwd_own_block(qc.data_ptr(), qs.data_ptr(), kc.data_ptr(), ks.data_ptr(),
                                                  vt.data_ptr(), vta.data_ptr(), B, S, Hq, Hkv, D, w.scale,
                                                  oo.data_ptr(), lo.data_ptr(), sh),
                lambda: L.mxfa_lse_merge(oc.data_ptr(), lc.data_ptr(), oo.data_ptr(), lo.data_ptr(), B, S, Hq, D,
                                         out.data_ptr(), *ov[4:], mx.OUT_BF16, lse.data_ptr(), sh),
            ]
        for i, c in enumerate(calls):
            if evs is not None:
                evs[i][0].record(stream)
            st = c()
            if st != 0:
                raise mx.MxfaError(st, L.mxfa_last_error().decode())
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per = {n: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]))
           for i, n in enumerate(names)}

    flops = 2.0 * B * Hq * S * S * D
    comp_flops = 512.0 * completed_pairs(B, Hq, S)
    own_flops = 512.0 * own_pairs(B, Hq, S)
    attn_name = "fused" if fused else "leaky" if leaky else "fused_mxfp8" if mx8 else "completed"
    attn_flops = comp_flops + own_flops if (fused or leaky or mx8) else comp_flops
    achieved = attn_flops / (per[attn_name] * 1e-3) / 1e12
    n_q, n_kv = B * Hq * S, B * Hkv * S
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    kernels = {} if fused else {
        "quantize_q": {"ms": per["quantize_q"], "GB/s": gbs(n_q * D * (2 + 1 + 1 / 32), per["quantize_q"])}}
    kernels |= {
        "quantize_kv": {"ms": per["quantize_kv"],
                        "GB/s": gbs(n_kv * D * ((2 + 1 + 1 / 32) + (2 + 1 + 1 / 32 + 1 + 1 / 128)), per["quantize_kv"])},
    }
    if fused or leaky or mx8:
        kernels[attn_name] = {"ms": per[attn_name], "TFLOP/s": achieved, "algorithmic_flop": attn_flops}
    else:
        kernels["completed"] = {"ms": per["completed"], "TFLOP/s": achieved, "algorithmic_flop": comp_flops}
        kernels["own_block"] = {"ms": per["own_block"], "TFLOP/s": own_flops / (per["own_block"] * 1e-3) / 1e12,
                                "GB/s": gbs(n_q * (D + 4 + D * 4 + 4) + n_kv * 2 * (D + 4), per["own_block"])}
        kernels["merge"] = {"ms": per["merge"], "GB/s": gbs(n_q * (2 * D * 4 + 2 * 4 + D * 2 + 4), per["merge"])}
    src = os.path.join(ROOT, "causal_mxfp8_block_amd", "csrc", "attn_completed.hip")
    traffic = read_traffic(src, attn_name) if w.name == "gqa16x4_s32k_amplitudes" else None
    value = flops / (ms_step * 1e-3) / 1e12
    measured_peak = measure_mfma_peak(torch)
    pages_ms = PAGES_OWN_BLOCK_MS.get((Hq, Hkv, S)) if (lay == "bshd" and B == 1 and args.path == "fused") else None
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / (flops / (pages_ms * 1e-3) / 1e12), 4) if pages_ms else None,
        "dtype": "mxfp8",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "D": D, "layout": lay,
                   "causal": True, "values": w.values, "output": "mxfp8" if mx8 else "bf16", "path": args.path},
        "pct_mfma_peak": round(100.0 * value / MFMA_FP8_PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": f"attn_kernel ({attn_name})", "launch_ms": round(per[attn_name], 4),
                     "measured_peak": round(measured_peak, 1),
                     "frac_of_measured_peak": round(achieved / measured_peak, 4)},
        "kernels": {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in d.items()}
                    for n, d in kernels.items()},
        "cpu_baseline": None,
    }
    if args.cpu_rows > 0 and not leaky:  # the baseline times the oracle of the leak-free path
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows)
    print(json.dumps(res), flush=True)


def run_fwdbwd(args, torch, mx, WORKLOADS, make_inputs):
    """One step = quantise Q, K, V; fused forward; backward on decoded operands (its preparation,
    dK/dV and dQ kernels) for a seeded dO. Prints one JSON line."""
    name = "mha16_s32k_sbhd" if args.workload == "gqa16x4_s32k_amplitudes" else args.workload
    w = WORKLOADS[name]
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = to(inp.q), to(inp.k), to(inp.v)
    rng = np.random.default_rng(w.seed + 1)
    g = torch.from_numpy(rng.standard_normal(inp.q.shape).astype(np.float32)).to(dev).to(torch.bfloat16)
    lay, B, S, Hq, Hkv, D = w.layout, w.B, w.S, w.Hq, w.Hkv, w.D
    stream = torch.cuda.current_stream(dev)
    ws_b = torch.empty(int(mx.lib().mxfa_attn_bwd_workspace_bytes(B, S, Hq, Hkv, D)), dtype=torch.uint8, device=dev)
    names = ["quantize", "forward", "backward"]

    def step(evs=None):
        def rec(i, j):
            if evs is not None:
                evs[i][j].record(stream)
        rec(0, 0)
        qc, qs = mx.mxfp8_quantize(q, "rowwise", lay)
        kc, ks, vc, vcs, vt, vta = mx.mxfp8_quantize_kv(k, v, lay)
        rec(0, 1)
        rec(1, 0)
        o, lse = mx.attn_fwd_fused(qc, qs, kc, ks, vc, vcs, vt, vta, w.scale, layout=lay)
        rec(1, 1)
        rec(2, 0)
        mx.attn_bwd(qc, qs, kc, ks, vt, vta, o, lse, g, w.scale, layout=lay, workspace=ws_b)
        rec(2, 1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per = {n: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]))
           for i, n in enumerate(names)}
    fwd_flops = 2.0 * B * Hq * S * S * D
    value = 3.5 * fwd_flops / (ms_step * 1e-3) / 1e12
    # algorithmic backward work: 5 products of 2*D FLOP (S, dP, dV, dK, dQ) per (query, visible key) pair
    bwd_alg = 1280.0 * (completed_pairs(B, Hq, S) + own_pairs(B, Hq, S))
    res = {
        "metric": METRIC_FWDBWD, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": round(value / PAGES_FWDBWD_TFLOPS, 4) if w.name == "mha16_s32k_sbhd" else None,
        "dtype": "mxfp8 fwd / bf16 bwd", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "D": D, "layout": lay, "causal": True,
                   "values": w.values, "flop_count": "FlashAttention convention: fwd 2BHS^2D, bwd 2.5x fwd"},
        "roofline": {"bound": "mfma", "achieved": round(bwd_alg / (per["backward"] * 1e-3) / 1e12, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_alg / (per["backward"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "backward (preparation + dK/dV + dQ kernels, bf16 MFMA)",
                     "launch_ms": round(per["backward"], 4)},
        "kernels": {n: {"ms": round(per[n], 4)} for n in names},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
