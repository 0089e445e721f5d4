"""Host-side accounting of bench.py (no GPU): the algorithmic work and the
band efficiency reported on the catch-up line."""
import random

import bench


def brute_band(avail, p0, n, W=750, qtile=128, qw=32):
    """Score blocks by enumeration: a wave's 32-key half-tile of the absolute
    64-key grid is computed when any of its queries sees any of its keys."""
    visible = computed = 0
    for qc in range(0, n, qtile):
        qs = list(range(p0 + qc, p0 + min(n, qc + qtile)))
        lo = max(avail, qs[0] - W + 1)
        hi = qs[-1]
        t0 = (lo // 64) * 64
        for w in range(0, len(qs), qw):
            wq = qs[w:w + qw]
            keys = set()
            for q in wq:
                ks = range(max(avail, q - W + 1), q + 1)
                visible += len(ks)
                keys.update(ks)
            for kb in range(t0, hi + 1, 32):
                if any(kb <= k < kb + 32 for k in keys):
                    computed += 32 * qw
    return visible, computed


def test_band_matches_enumeration_and_work():
    rng = random.Random(7)
    for _ in range(25):
        avail = rng.randrange(0, 3000)
        nkv = rng.randrange(0, 1000)
        n = rng.choice([32, 33, 100, 128, 129, 300, 512])
        v, c = bench.mfma_band(avail, avail + nkv, n)
        assert (v, c) == brute_band(avail, avail + nkv, n)
        # the visible pairs are the ones the flop count uses
        assert 4 * bench.D * bench.H * v == bench.attn_work(nkv, n)[1]
        assert c % 1024 == 0 and c >= v


def test_band_full_window_value():
    # 512 queries with 749 old keys: 0.9375 of the computed pairs are visible
    v, c = bench.mfma_band(1000, 1750, 512)
    assert (v, c) == (384000, 409600)


def test_more_than_one_gpu_is_refused_before_any_device_work():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
