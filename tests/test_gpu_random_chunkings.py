"""Seeded random chunkings on each arithmetic path, through the C ABI.

Chunk invariance holds per arithmetic path (the path of a sub-batch is a
pure function of the cache description and its size): fp32 always takes the
vector kernel; bf16 sub-batches under 32 frames take the vector kernel, from
32 frames on the matrix-core kernel.  So every random schedule here keeps
all of its sub-batches on one path and must reproduce, bit for bit, a
reference on the same path: the offline pass (whose 512-frame sub-batches
take the matrix path for bf16, the vector path for fp32) or, for the bf16
vector path, 4-frame feeds.  Sizes cross the 512-frame split, and the
sequences cross compactions of the 1536-slot ring at unaligned start
positions; the modulo ring must give the same bits as the compacting ring
(streaming plan, "Unbounded length" and SHIPPED, Verification: incremental
equals offline)."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt

from gpu_util import DEV, Pool, empty, host, run_feeds, say, seqs, stream, to_dev

pytestmark = pytest.mark.gpu


def offline(desc, q, k, v, T, start):
    sb = vrt.offline_scratch_bytes(desc, T)
    scratch = torch.empty(sb, dtype=torch.uint8, device=DEV)
    out = empty((T, q.shape[-2], q.shape[-1]), desc.dtype)
    vrt.enc_attn_offline(desc, q, k, v, T, start, out, scratch, sb, stream())
    torch.cuda.synchronize()
    return host(out)


def random_sizes(rng, lo, hi, T):
    sizes, t = [], 0
    while t < T:
        m = int(rng.integers(lo, hi + 1))
        sizes.append(m)
        t += m
    return sizes


def matrix_sizes(rng, T):
    """Feed sizes that tile T exactly with every sub-batch of at least 32
    frames: parts of 32 .. 700 frames, none of 513 .. 543 (its 512-frame
    split would leave under 32), and never a remainder under 32."""
    def ok(m, left):
        return 32 <= m <= left and not (512 < m < 544) and m <= 700 and (m == left or left - m >= 32)
    sizes, left = [], T
    while left > 0:
        for _ in range(1000):
            m = int(rng.integers(32, 701))
            if ok(m, left):
                break
        else:
            m = left if ok(left, left) else left - 32
        assert ok(m, left)
        sizes.append(m)
        left -= m
    return sizes


def feed(pool, starts, qd, kd, vd, sizes):
    for s, st in enumerate(starts):
        pool.states[s].reset(st)
    return host(run_feeds(pool, range(len(starts)), 0, qd.shape[1], qd, kd, vd, sizes))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_fp32_random_chunkings_equal_offline(seed):
    S, L, T, H, d = 2, 1, 1700, 20, 64
    rng = np.random.default_rng([seed, 11])
    starts = [int(x) for x in rng.integers(0, 1_000_000, S)]
    desc = vrt.enc_desc(dtype=vrt.F32, n_layers=L)
    q, k, v = seqs(40 + seed, S, L, T, H, d, 1.0, vrt.F32)
    qd, kd, vd = (to_dev(x, vrt.F32) for x in (q, k, v))
    pool = Pool(desc, S, starts)
    refs = [offline(desc, qd[s, 0], kd[s, 0], vd[s, 0], T, starts[s]) for s in range(S)]
    for trial in range(3):
        sizes = random_sizes(rng, 1, 600, T)
        say(f"fp32 seed {seed} trial {trial}: {len(sizes)} feeds, sizes {sizes[:8]}...")
        out = feed(pool, starts, qd, kd, vd, sizes)
        for s in range(S):
            assert np.array_equal(out[s, 0], refs[s]), (seed, trial, s, sizes)
    pool.close()


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_bf16_vector_path_random_chunkings(seed):
    S, L, T, H, d = 3, 2, 1700, 20, 64
    rng = np.random.default_rng([seed, 12])
    starts = [int(x) for x in rng.integers(0, 1_000_000, S)]
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=L)
    q, k, v = seqs(50 + seed, S, L, T, H, d, 0.5, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    pool = Pool(desc, S, starts)
    ref = feed(pool, starts, qd, kd, vd, [4])
    for trial in range(2):
        sizes = random_sizes(rng, 1, 31, T)
        say(f"bf16 vector seed {seed} trial {trial}: {len(sizes)} feeds")
        assert all(vrt.attn_path(desc, m) == vrt.attn_path(desc, 4) for m in set(sizes))
        out = feed(pool, starts, qd, kd, vd, sizes)
        assert np.array_equal(out, ref), (seed, trial, sizes)
    pool.close()


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_bf16_matrix_path_random_chunkings_equal_offline(seed):
    S, L, T, H, d = 2, 2, 2600, 20, 64
    rng = np.random.default_rng([seed, 13])
    starts = [int(x) for x in rng.integers(0, 1_000_000, S)]
    q, k, v = seqs(60 + seed, S, L, T, H, d, 1.0, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=L)
    mod = vrt.enc_desc(dtype=vrt.BF16, n_layers=L, kind=vrt.ENC_MODRING)
    refs = [[offline(desc, qd[s, l], kd[s, l], vd[s, l], T, starts[s]) for l in range(L)] for s in range(S)]
    pools = {"compacting": Pool(desc, S, starts), "modulo": Pool(mod, S, starts)}
    for trial in range(2):
        sizes = matrix_sizes(rng, T)
        assert sum(sizes) == T
        say(f"bf16 matrix seed {seed} trial {trial}: sizes {sizes}")
        assert all(vrt.attn_path(desc, min(m, 512)) == vrt.attn_path(desc, 512) for m in set(sizes))
        for name, pool in pools.items():
            out = feed(pool, starts, qd, kd, vd, sizes)
            for s in range(S):
                for l in range(L):
                    assert np.array_equal(out[s, l], refs[s][l]), (name, seed, trial, s, l, sizes)
    for pool in pools.values():
        pool.close()
