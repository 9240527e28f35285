"""The longest sequence the library accepts, S = 2^24 (B = 1, one query and one KV head, D = 128).

At this length every offset the forward kernels form reaches its largest value: K rows end 2^31
bytes into a head, V columns start up to 127 S bytes in, and the buffer records hold 2^31 bytes. The
oracle cannot compute a row of this length in test time (each row reads 2^24 keys), so the inputs
repeat with a period of P = 4320 tokens (135 blocks of 32: the MXFP8 blocks of V and of P then repeat
too, and no power-of-two offset error is a multiple of P). Two properties that hold at any size turn
the oracle's rows of a 2P-token problem into the expected rows of the long one:

- causality: row i < P sees only keys j <= i, the same keys as in the short problem;
- periodicity: for row i = mP + r, the completed keys j < 32 floor(i/32) are m whole periods plus the
  completed keys of row r, so its unnormalised sums are m (E_{P+r} - E_r) + E_r with E the
  exponentiated log-sum-exp (times O for the numerator) of the short problem's rows P + r and r; its
  own block equals row r's. The merge is then the oracle's own merge.

The quantisers are checked on every element: the first period against the oracle, the rest by the
repetition itself. Gate: TE#3865 "Testing" asks for end-to-end numerics; the tolerance is the forward
gate's 2e-2 * RMS per row group (start, middle, end). A CPU test checks the composition itself: at a
length the oracle computes directly, the composed rows equal the oracle's own."""
import numpy as np
import pytest
import torch

import oracle
import causal_mxfp8_block_amd as mx
from causal_mxfp8_block_amd.inputs import custom, make_inputs
from gpu_helpers import DEV, gate, say

S = 1 << 24
P = 4320
TOL = 2e-2


def _rows(seed=5):
    rng = np.random.default_rng(seed)
    mid = [S // 2 - 33, S // 2 - 32, S // 2 - 1, S // 2, S // 2 + 31]
    end = [S - 4 * P - 1, S - P, S - 65, S - 33, S - 32, S - 31, S - 2, S - 1]
    end += sorted(rng.integers(S - 8 * P, S, size=4).tolist())
    return {"start": np.arange(0, 64), "middle": np.array(mid), "end": np.array(sorted(set(end)))}


def _repeats(x: torch.Tensor, dim: int, period: int) -> bool:
    n = x.shape[dim]
    return torch.equal(x.narrow(dim, period, n - period), x.narrow(dim, 0, n - period))


def _tile_to(x: torch.Tensor, dim: int, n: int) -> torch.Tensor:
    reps = [1] * x.dim()
    reps[dim] = -(-n // x.shape[dim])
    return x.repeat(*reps).narrow(dim, 0, n).contiguous()


def expected_rows(views, z, scale, rows, period):
    """Expected O, lse, allowance and its hardware terms of the given rows of a sequence whose inputs
    repeat every ``period`` tokens (a multiple of 32), from the oracle's rows of the two-period problem
    ``views`` (its quantisation ``z``): rows below the period directly (causality), later rows
    composed from rows r and period + r (periodicity; no allowance: one code's share of m periods)."""
    m = rows // period
    r = rows % period
    late = rows >= period
    orows = np.unique(np.concatenate([rows[~late], r[late], period + r[late]])).astype(np.int32)
    ro, rl, parts = oracle.forward(*views, scale, orows, quant=z)
    at = {int(x): i for i, x in enumerate(orows)}
    D = ro.shape[-1]
    ref = np.empty((len(rows), D))
    rlse = np.empty(len(rows))
    allow = np.zeros((len(rows), D))
    hw = np.zeros((len(rows), D))
    for n, i in enumerate(rows):
        if i < period:
            j = at[int(i)]
            ref[n], rlse[n] = ro[0, 0, j], rl[0, 0, j]
            allow[n] = parts["allowance"][0, 0, j]
            hw[n] = parts["allowance_code"][0, 0, j] + parts["allowance_pv"][0, 0, j]
            continue
        a, b = at[int(period + r[n])], at[int(r[n])]
        o1, l1 = parts["o_c"][0, 0, a], parts["lse_c"][0, 0, a]
        orr, lr = parts["o_c"][0, 0, b], parts["lse_c"][0, 0, b]
        er = 0.0 if np.isneginf(lr) else np.exp(lr - l1)
        den = m[n] * (1.0 - er) + er
        oc = (m[n] * (o1 - er * orr) + er * orr) / den
        lc = l1 + np.log(den)
        o, l_ = oracle.lse_merge(oc[None], np.array([lc]), parts["o_o"][0, 0, b][None],
                                 np.array([parts["lse_o"][0, 0, b]]))
        ref[n], rlse[n] = o[0], l_[0]
    return ref, rlse, allow, hw


def test_periodic_composition_equals_the_oracle():
    """CPU: at a length the oracle computes directly (five periods of 128 and part of a sixth), the
    composed rows equal the oracle's own rows of the long problem."""
    per, n = 128, 5 * 128 + 96
    base = make_inputs(custom(1, 1, 1, per, seed=6, name="period"))
    two = [oracle.BF16View.bshd(np.tile(getattr(base, x), (1, 2, 1, 1))) for x in ("q", "k", "v")]
    reps = -(-n // per)
    full = [oracle.BF16View.bshd(np.ascontiguousarray(np.tile(getattr(base, x), (1, reps, 1, 1))[:, :n]))
            for x in ("q", "k", "v")]
    rows = np.array([0, 31, 32, 100, 127, 128, 130, 160, 255, 256, 300, 511, 513, 640, 660, 700, 720, n - 1])
    scale = base.workload.scale
    ref, rlse, _, _ = expected_rows(two, oracle.quantize_all(*two), scale, rows, per)
    ro, rl, _ = oracle.forward(*full, scale, rows.astype(np.int32))
    assert np.max(np.abs(ref - ro[0, 0])) <= 1e-12 * np.max(np.abs(ro))
    assert np.max(np.abs(rlse - rl[0, 0])) <= 1e-12


@pytest.mark.gpu
def test_forward_at_the_longest_sequence():
    base = make_inputs(custom(1, 1, 1, P, seed=2024, name="period"))
    w = base.workload
    say(f"longest sequence: B=1 Hq=Hkv=1 S={S} D=128 bshd, period {P} of N(0,1) tokens (seed {w.seed})")
    # the short problem (two periods) for the oracle, the long one on the device
    short = [np.tile(getattr(base, n), (1, 2, 1, 1)) for n in ("q", "k", "v")]
    views = [oracle.BF16View.bshd(x) for x in short]
    dev = [_tile_to(torch.from_numpy(getattr(base, n).view(np.int16)).to(DEV), 1, S).view(torch.bfloat16)
           for n in ("q", "k", "v")]
    q, k, v = dev

    say("quantisers at S = 2^24")
    z = oracle.quantize_all(*views)
    got = {}
    got["qc"], got["qs"] = mx.mxfp8_quantize(q, "rowwise")
    got["kc"], got["ks"] = mx.mxfp8_quantize(k, "rowwise")
    got["vc"], got["vcs"], got["vt"], got["vta"] = mx.mxfp8_quantize(v, "v")
    torch.cuda.synchronize()
    # token axis and period of each output ([B,H,S,.], col codes [B,H,D,S], col scales [B,H,S/32,D])
    axis = {"qc": 2, "qs": 2, "kc": 2, "ks": 2, "vc": 3, "vcs": 2, "vt": 2, "vta": 2}
    for key, a in axis.items():
        g = got[key]
        per = P // 32 if key == "vcs" else P
        first = g.narrow(a, 0, per).cpu().numpy()
        want = np.take(getattr(z, key), np.arange(per), axis=a)
        assert np.array_equal(first, want), f"{key}: first period differs from the oracle"
        assert _repeats(g, a, per), f"{key}: does not repeat with the input's period"
    del got
    torch.cuda.empty_cache()

    say("whole forward at S = 2^24 (attn_fwd)")
    out, lse = mx.attn_fwd(q, k, v, w.scale, layout="bshd", out_dtype=torch.float32)
    torch.cuda.synchronize()
    groups = _rows()
    rows = np.concatenate(list(groups.values()))
    ridx = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    go = out[0, :, 0, :].index_select(0, ridx).double().cpu().numpy()
    gl = lse[0, 0].index_select(0, ridx).double().cpu().numpy()
    del out, lse, dev, q, k, v
    torch.cuda.empty_cache()

    say("oracle rows of the two-period problem")
    ref, rlse, allow, hw = expected_rows(views, z, w.scale, rows, P)

    off = 0
    for name, rr in groups.items():
        sl = slice(off, off + len(rr))
        off += len(rr)
        rms = float(np.sqrt(np.mean(ref[sl] ** 2)))
        gate(f"S=2^24 {name} rows", go[None, None, sl], ref[None, None, sl], rms, rr,
             allowance=allow[None, None, sl], allowance_hw=hw[None, None, sl], tol=TOL, max_over_frac=2e-3)
    assert np.max(np.abs(gl - rlse)) < 1e-3
