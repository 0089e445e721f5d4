"""GPU A/B of the encoder cache stored as a modulo ring (ENC_MODRING: slot =
position % ring_slots, no compaction) against the compacting ring (ENC_RING),
the way the pages validate their decoder ring against a buffer that never
wraps.  The kernels see the same keys at the same absolute positions and
only address them differently, so the bar is bit-identity: outputs, and the
ring rows of every position still in the window.  Sampled rows are also
checked against the fp64 oracle (gpu_util tolerances)."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention
from oracle.ring import DecRing, EncRing

from gpu_util import Pool, check_close, host, run_feeds, say, seqs, to_dev

pytestmark = pytest.mark.gpu
THETA = 1.0e6
W = 750


def _ab(dtype, S, L, T, starts, sizes, seed, scale):
    H, d = 20, 64
    q, k, v = seqs(seed, S, L, T, H, d, scale, dtype)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    res = {}
    for kind in (vrt.ENC_RING, vrt.ENC_MODRING):
        desc = vrt.enc_desc(dtype=dtype, n_layers=L, kind=kind)
        pool = Pool(desc, S, starts)
        say(f"  kind {kind}: ring {desc.ring_slots}, feeds {sizes[:6]}")
        res[kind] = (host(run_feeds(pool, range(S), 0, L, qd, kd, vd, sizes)), pool)
    ring_out, rp = res[vrt.ENC_RING]
    mod_out, mp = res[vrt.ENC_MODRING]
    assert np.array_equal(ring_out, mod_out)
    for s in range(S):
        r = EncRing()
        r.reset(starts[s])
        m = DecRing(slots=mp.desc.ring_slots)
        m.reset(starts[s])
        t, i = 0, 0
        while t < T:
            n = min(sizes[i % len(sizes)], T - t)
            r.feed(n)
            m.append(n)
            t, i = t + n, i + 1
        for l in range(L):
            assert rp.states[s].query(l) == (r.abs_base, r.n_kv)
            assert mp.states[s].query(l) == (starts[s], T)
        # the last W positions: ring slot p - abs_base vs modulo slot p % slots
        p_hi = starts[s] + T
        for l in range(L):
            for which, head in ((0, 0), (1, 7), (0, 19)):
                for p in range(p_hi - W, p_hi, 37):
                    a = rp.ring_bytes(s, l, which, head, p - r.abs_base, p - r.abs_base + 1)
                    b = mp.ring_bytes(s, l, which, head, m.slot(p), m.slot(p) + 1)
                    assert a == b, (s, l, which, head, p)
    rp.close()
    mp.close()
    return q, k, v, mod_out


def test_modring_vector_path_bit_identical():
    """4-frame feeds (vector path, fused append), bf16, 3 streams x 2 layers,
    2000 frames (two compactions in the compacting ring; the modulo ring of
    1280 slots wraps once), unaligned starts."""
    starts = [0, 1234, 987_655]
    q, k, v, out = _ab(vrt.BF16, 3, 2, 2000, starts, [4], 50, 0.5)
    ts = [0, 3, 749, 750, 1279, 1280, 1281, 1535, 1536, 1537, 1999]
    for s in (0, 2):
        ref = attention.windowed_at(q[s, 1], k[s, 1], v[s, 1], starts[s], W, THETA, ts)
        check_close(out[s, 1][ts], ref, vrt.BF16, f"modring stream {s} sampled")


def test_modring_fp32_vector_path_bit_identical():
    """fp32 storage, 4- and 7-frame feeds, 1 stream x 1 layer, 1700 frames."""
    q, k, v, out = _ab(vrt.F32, 1, 1, 1700, [77], [4, 7], 51, 1.0)
    ref = attention.windowed(q[0, 0], k[0, 0], v[0, 0], 77, W, THETA)
    check_close(out[0, 0], ref, vrt.F32, "modring fp32 all rows")


def test_modring_matrix_path_bit_identical():
    """512-frame and mixed feeds (matrix path, separate append), bf16, 2
    streams x 2 layers, 3000 frames; a start near the top of the position
    range checks the modulo of large tile positions."""
    starts = [5, 2 ** 31 - 3000]
    for sizes in ([512], [37, 300, 64, 512, 33, 129]):
        q, k, v, out = _ab(vrt.BF16, 2, 2, 3000, starts, sizes, 52, 1.0)
    ts = [0, 511, 512, 1023, 1279, 1280, 1536, 2047, 2559, 2999]
    for s in range(2):
        ref = attention.windowed_at(q[s, 0], k[s, 0], v[s, 0], starts[s], W, THETA, ts)
        check_close(out[s, 0][ts], ref, vrt.BF16, f"modring matrix stream {s} sampled")


def test_modring_offline_equals_stream():
    """The offline pass needs no ring; a modulo-ring stream of 512-frame feeds
    equals it bit for bit."""
    desc = vrt.enc_desc(n_layers=1, kind=vrt.ENC_MODRING)
    T, H, d, start = 2100, 20, 64, 4321
    q, k, v = seqs(53, 1, 1, T, H, d, 1.0, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    pool = Pool(desc, 1, [start])
    say("modring: 512-frame feeds vs offline")
    out = host(run_feeds(pool, [0], 0, 1, qd, kd, vd, [512]))[0, 0]
    sb = vrt.offline_scratch_bytes(desc, T)
    scratch = torch.empty(sb, dtype=torch.uint8, device=qd.device)
    off = torch.empty_like(qd[0, 0])
    vrt.enc_attn_offline(desc, qd[0, 0], kd[0, 0], vd[0, 0], T, start, off, scratch, sb,
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(out, host(off))
    pool.close()
