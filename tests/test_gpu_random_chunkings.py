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
equals offline).  The lookahead windows and the conv stem get the same
treatment (moonshine map, "Per-layer sliding-window mask"; streaming plan,
"Chunk alignment")."""
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


@pytest.mark.parametrize("seed", [0, 1])
def test_lookahead_random_chunkings_equal_offline(seed):
    """(left, right) windows without rotation always take the vector kernel,
    so any schedule of feed sizes answers each query with the offline pass's
    bits (the moonshine streaming head: 8 x 40, windows (16, 4))."""
    S, L, T, H, d, right = 2, 2, 700, 8, 40, 4
    rng = np.random.default_rng([seed, 14])
    starts = [int(x) for x in rng.integers(0, 1_000_000, S)]
    desc = vrt.lookahead_desc(16, right, dtype=vrt.BF16, n_layers=L, heads=H, head_dim=d)
    q, k, v = seqs(70 + seed, S, L, T, H, d, 1.0, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    f = right - 1
    refs = [[offline(desc, qd[s, l], kd[s, l], vd[s, l], T, starts[s])[:T - f] for l in range(L)]
            for s in range(S)]
    for trial in range(3):
        sizes = random_sizes(rng, 1, 300, T)
        say(f"lookahead seed {seed} trial {trial}: {len(sizes)} feeds")
        pool = Pool(desc, S, starts)
        states = [pool.states[i] for i in range(S)]
        outs, t = [], 0
        for m in sizes:
            m = min(m, T - t)
            _, nkv = states[0].query(0)
            n_out = vrt.attn_out_frames(desc, nkv, m)
            qc, kc, vc = (x[:, :, t:t + m].contiguous() for x in (qd, kd, vd))
            oc = torch.empty_like(qc)
            vrt.enc_attn_feed(states, 0, L, qc, kc, vc, m, oc, stream())
            if n_out:
                outs.append(oc[:, :, :n_out].clone())
            t += m
        torch.cuda.synchronize()
        got = host(torch.cat(outs, dim=2))
        pool.close()
        for s in range(S):
            for l in range(L):
                assert np.array_equal(got[s, l], refs[s][l]), (seed, trial, s, l, sizes)


@pytest.mark.parametrize("seed", [0, 1])
def test_conv_stem_random_chunkings_equal_one_feed(seed):
    """The causal conv stem: every output row's k order is fixed, so any
    schedule of mel chunk sizes (odd ones change how many conv0 frames are
    carried between feeds) gives the one-feed bits."""
    import synth
    n_mel, dm, S, T = 128, 1280, 2, 90
    rng = np.random.default_rng([seed, 15])
    w = synth.conv_weights(72 + seed, n_mel, dm)
    bfd = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16)
    tap_major = lambda W_: np.ascontiguousarray(np.transpose(W_, (0, 2, 1)).reshape(W_.shape[0], -1))
    tens = {"w0": bfd(tap_major(w["w0"])), "b0": bfd(w["b0"]), "w1": bfd(tap_major(w["w1"])), "b1": bfd(w["b1"])}
    cw = vrt.conv_weights(tens["w0"], tens["b0"], tens["w1"], tens["b1"])
    mel = bfd(np.stack([synth.mel_frames(73 + seed, s, T, n_mel) for s in range(S)]))
    nb = vrt.conv_stem_device_bytes(n_mel, dm)

    def run(sizes):
        mem = torch.empty(S * nb, dtype=torch.uint8, device=DEV)
        stems = [vrt.ConvStem(n_mel, dm, mem[i * nb:(i + 1) * nb], nb) for i in range(S)]
        outs, t = [], 0
        for m in sizes:
            m = min(m, T - t)
            n_out = stems[0].out_frames(m)
            wsb = vrt.conv_workspace_bytes(n_mel, dm, S, m)
            ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
            o = torch.empty((S, max(n_out, 1), dm), dtype=torch.bfloat16, device=DEV)
            assert vrt.conv_stem_feed(stems, mel[:, t:t + m].contiguous(), m, cw, o, ws, wsb, stream()) == n_out
            if n_out:
                outs.append(o[:, :n_out].clone())
            t += m
        torch.cuda.synchronize()
        res = host(torch.cat(outs, dim=1))
        for st in stems:
            st.close()
        return res

    ref = run([T])
    for trial in range(3):
        sizes = random_sizes(rng, 1, 25, T)
        say(f"conv stem seed {seed} trial {trial}: sizes {sizes}")
        assert np.array_equal(run(sizes), ref), (seed, trial, sizes)


@pytest.mark.parametrize("seed", [0, 1])
def test_block_random_chunkings(seed):
    """The attention half of an encoder block (RMSNorm, q/k/v, the path,
    output projection and residual): the norm and projections are row-local
    and the projections' k order is fixed, so after the same 750-frame
    pre-fill any schedule of feeds under 32 frames reproduces 4-frame feeds,
    and any schedule that keeps every sub-batch on the matrix path
    reproduces 512-frame feeds, bit for bit, across compactions."""
    import synth
    from oracle import block
    S, T, dim = 2, 1700, 1280
    rng = np.random.default_rng([seed, 16])
    starts = [int(x) for x in rng.integers(0, 1_000_000, S)]
    wts = synth.block_weights(80 + seed, 0, dim)
    bfd = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16)
    wd = {k: bfd(v) for k, v in wts.items()}
    w_qkv = torch.cat([wd["wq"], wd["wk"], wd["wv"]], 0).contiguous()
    bw = vrt.block_weights(wd["norm_w"], w_qkv, wd["bq"], wd["bv"], wd["wo"], wd["bo"], block.EPS)
    xd = bfd(np.stack([synth.block_input(81 + seed, s, 0, T, dim) for s in range(S)]))
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=1)

    def run(sizes):
        pool = Pool(desc, S, starts)
        out = torch.empty_like(xd)
        t = 0
        for m in sizes:
            m = min(m, T - t)
            if m <= 0:
                break
            wsb = vrt.block_workspace_bytes(desc, S * m)
            ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
            xc = xd[:, t:t + m].contiguous()
            oc = torch.empty_like(xc)
            vrt.enc_block_feed(pool.states, 0, xc, m, bw, oc, ws, wsb, stream())
            out[:, t:t + m] = oc
            t += m
        assert t == T
        torch.cuda.synchronize()
        pool.close()
        return host(out)

    vec_ref = run([750] + [4] * 238)
    mat_ref = run([512] * 4)
    for trial in range(2):
        vs = [750] + random_sizes(rng, 1, 31, T - 750)
        say(f"block seed {seed} trial {trial}: vector-path feeds after the pre-fill ({len(vs) - 1})")
        assert np.array_equal(run(vs), vec_ref), (seed, trial, vs)
        ms = matrix_sizes(rng, T)
        say(f"block seed {seed} trial {trial}: matrix-path feeds {ms}")
        assert np.array_equal(run(ms), mat_ref), (seed, trial, ms)
