"""GPU parity of the matrix-core (catch-up) path: bf16 sub-batches of 32 or
more frames run k_attn_mfma after a separate RoPE + append launch.

Bar: bit-identical outputs under every chunking whose sub-batches all take
this path (feeds of 512, 100, mixed sizes >= 32, and the offline pass), ring
metadata equal to the oracle's ring model, and max-abs error <= 2e-2 against
the fp64 oracle (gpu_util.BF16_TOL) on the rows checked.  Sizes are chosen so
that every sub-batch, including the last one of each run, has >= 32 frames."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention
from oracle.ring import EncRing

from gpu_util import DEV, Pool, check_close, empty, host, run_feeds, say, seqs, stream, to_dev

pytestmark = pytest.mark.gpu
THETA = 1.0e6
W = 750


def offline(desc, q, k, v, T, start):
    sb = vrt.offline_scratch_bytes(desc, T)
    scratch = torch.empty(sb, dtype=torch.uint8, device=DEV)
    out = empty((T, q.shape[-2], q.shape[-1]), desc.dtype)
    vrt.enc_attn_offline(desc, q, k, v, T, start, out, scratch, sb, stream())
    torch.cuda.synchronize()
    return host(out)


def ring_model(start, sizes, T):
    r = EncRing()
    r.reset(start)
    t, i = 0, 0
    while t < T:
        m = min(sizes[i % len(sizes)], T - t)
        r.feed(m)
        t += m
        i += 1
    return r


def test_path_is_mfma_for_these_sizes():
    d = vrt.enc_desc(dtype=vrt.BF16)
    for n in (32, 33, 100, 127, 128, 129, 130, 512):
        assert vrt.attn_path(d, n) == 1, n
    for n in (1, 4, 31):
        assert vrt.attn_path(d, n) == 0, n


def test_catchup_any_chunking_offline_and_oracle():
    """2 streams x 2 layers, bf16 N(0,1), unaligned starts, 2600 frames:
    512-frame feeds (compactions before sub-batches 4 and 5), 100-frame feeds,
    a mixed schedule of sizes >= 32 and the offline pass are bit-identical;
    the ring metadata follows the oracle's ring model; sampled rows (tile,
    query-tile and compaction boundaries) match the oracle."""
    S, L, T, H, d = 2, 2, 2600, 20, 64
    starts = [1234, 1_000_037]
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=L)
    q, k, v = seqs(30, S, L, T, H, d, 1.0, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    pool = Pool(desc, S, starts)
    runs = {}
    for sizes in ([512], [100], [37, 300, 64, 512, 33, 129]):
        for s in range(S):
            pool.states[s].reset(starts[s])
        say(f"mfma path: feeds {sizes}")
        runs[tuple(sizes)] = host(run_feeds(pool, range(S), 0, L, qd, kd, vd, sizes))
        for s in range(S):
            r = ring_model(starts[s], sizes, T)
            for l in range(L):
                assert pool.states[s].query(l) == (r.abs_base, r.n_kv), (sizes, s, l)
    base = runs[(512,)]
    for key, out in runs.items():
        assert np.array_equal(out, base), key
    for s in range(S):
        for l in range(L):
            say(f"offline stream {s} layer {l}")
            off = offline(desc, qd[s, l], kd[s, l], vd[s, l], T, starts[s])
            assert np.array_equal(off, base[s, l]), (s, l)
    ts = sorted({0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 511, 512, 748, 749, 750, 751, 1023,
                 1024, 1535, 1536, 1537, 1600, 2047, 2048, 2559, 2560, 2598, 2599})
    for s in range(S):
        for l in range(L):
            ref = attention.windowed_at(q[s, l], k[s, l], v[s, l], starts[s], W, THETA, ts)
            check_close(base[s, l][ts], ref, vrt.BF16, f"stream {s} layer {l} sampled")
    pool.close()


def test_catchup_threshold_and_ragged_query_tiles():
    """Sub-batch sizes at the path threshold and around the 128-query tile
    (32, 33, 127, 128, 129, 130: tiles with 1 or 2 queries, waves with none),
    from an empty ring at position 0, at an unaligned large position and
    ending at the last position the library accepts (2^31 - 1):
    bit-identical to the offline pass; every row checked against the oracle."""
    H, d = 20, 64
    sizes = [32, 33, 127, 128, 129, 130, 64]
    T = sum(sizes) * 2
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=1)
    for start in (0, 987_655, 2 ** 31 - T):
        q, k, v = seqs(31, 1, 1, T, H, d, 1.0, vrt.BF16)
        qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
        pool = Pool(desc, 1, [start])
        say(f"threshold sizes from start {start}")
        out = host(run_feeds(pool, [0], 0, 1, qd, kd, vd, sizes))[0, 0]
        off = offline(desc, qd[0, 0], kd[0, 0], vd[0, 0], T, start)
        assert np.array_equal(out, off), start
        ref = attention.windowed(q[0, 0], k[0, 0], v[0, 0], start, W, THETA)
        check_close(out, ref, vrt.BF16, f"all {T} rows, start {start}")
        pool.close()


def test_paths_mixed_in_one_stream():
    """4-frame feeds (vector path, fused append) interleaved with 200-frame
    feeds (matrix path, separate append): keys written by either path are
    read by the other; every row within tolerance of the oracle."""
    H, d, start = 20, 64, 77
    sizes = [4] * 60 + [200] + [4] * 40 + [200, 200]
    T = sum(sizes)
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=1)
    q, k, v = seqs(32, 1, 1, T, H, d, 0.5, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    pool = Pool(desc, 1, [start])
    say(f"mixed vector / matrix sub-batches, {T} frames")
    out = host(run_feeds(pool, [0], 0, 1, qd, kd, vd, sizes))[0, 0]
    ref = attention.windowed(q[0, 0], k[0, 0], v[0, 0], start, W, THETA)
    check_close(out, ref, vrt.BF16, "mixed paths, all rows")
    pool.close()


def test_batched_equals_serial_mfma():
    S, T, H, d = 3, 1100, 20, 64
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=1)
    starts = [5, 400, 123_456]
    q, k, v = seqs(33, S, 1, T, H, d, 1.0, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    say("mfma batched: 3 states in one call")
    pb = Pool(desc, S, starts)
    batched = host(run_feeds(pb, range(S), 0, 1, qd, kd, vd, [220]))
    ps = Pool(desc, S, starts)
    for s in range(S):
        one = host(run_feeds(ps, [s], 0, 1, qd[s:s + 1], kd[s:s + 1], vd[s:s + 1], [220]))
        assert np.array_equal(one[0], batched[s]), s
    pb.close()
    ps.close()
