"""Host-side checks of bench.py's contract that need no GPU: more than one GPU is refused with a
message (this library has no multi-GPU path), and the FLOP counts it reports are the FlashAttention
causal convention and the exact pair counts of the method."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_pair_counts_match_brute_force():
    import bench
    for B, Hq, S in ((1, 1, 32), (2, 3, 96), (1, 2, 160)):
        comp = own = 0
        for i in range(S):
            n = 32 * (i // 32)  # completed keys of query i
            comp += n
            own += i - n + 1    # its own block's keys up to itself
        assert bench.completed_pairs(B, Hq, S) == B * Hq * comp
        assert bench.own_pairs(B, Hq, S) == B * Hq * own
        # every visible pair once: the exact count 4 B Hq D S(S+1)/2 of 512-FLOP pairs (D = 128)
        assert 512 * (comp + own) * B * Hq == 4 * B * Hq * 128 * S * (S + 1) // 2
    assert np.isclose(2.0 * 1 * 16 * 32768 ** 2 * 128, 4.398e12, rtol=1e-3)
