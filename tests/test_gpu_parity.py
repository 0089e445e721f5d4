"""GPU parity: the HIP path through the C ABI against the fp64 oracle, on
seeded inputs, plus the invariances the method promises (bit-identical
chunked vs offline, any chunking, batched vs serial, ring vs linear buffer).

Tolerances: fp32 max|d|/max|ref| <= 1e-5; bf16 max|d| <= 2e-2 (gpu_util)."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention, rope
from oracle.ring import EncRing
from synth import qkv, offsets

from gpu_util import (DEV, Pool, check_close, empty, host, run_feeds, say, seqs, stream, to_dev,
                      rel_err)

pytestmark = pytest.mark.gpu
THETA = 1.0e6


def test_c0_fp32_chunked_offline_oracle_and_compaction():
    """1 stream, 1 layer, fp32, 20 x 64, window 750, ring 1536: 250 feeds of 4
    frames with one explicit compaction after feed 200, vs one offline pass."""
    say("C0: fp32 1000 frames, 4-frame feeds, compaction after feed 200")
    desc = vrt.enc_desc(dtype=vrt.F32, n_layers=1)
    T, H, d = 1000, 20, 64
    q, k, v = seqs(0, 1, 1, T, H, d, 1.0, vrt.F32)
    pool = Pool(desc, 1, [0])
    qd, kd, vd = (to_dev(x, vrt.F32) for x in (q, k, v))
    snap = {}

    def compact():
        torch.cuda.synchronize()
        assert pool.states[0].query(0) == (0, 800)
        snap["k"] = pool.ring_bytes(0, 0, 0, 3, 50, 800)
        snap["v"] = pool.ring_bytes(0, 0, 1, 17, 50, 800)
        vrt.ring_compact(pool.states, 0, 1, stream())
        torch.cuda.synchronize()
        assert pool.states[0].query(0) == (50, 750)
        # compaction contents: byte-identical rows, moved to the front
        assert pool.ring_bytes(0, 0, 0, 3, 0, 750) == snap["k"]
        assert pool.ring_bytes(0, 0, 1, 17, 0, 750) == snap["v"]

    chunked = host(run_feeds(pool, [0], 0, 1, qd, kd, vd, [4], hooks={200: compact}))[0, 0]
    assert "k" in snap
    # ring model of the oracle: same schedule, same metadata
    r = EncRing()
    for i in range(250):
        if i == 200:
            r.compact()
        r.feed(4)
    assert pool.states[0].query(0) == (r.abs_base, r.n_kv)
    # ring contents vs the oracle's rotated keys / raw values
    kr = rope.apply(k[0, 0], np.arange(T), THETA)
    for h in (0, 11, 19):
        ring_k = pool.ring_rows(0, 0, 0, h, 0, r.n_kv)
        ring_v = pool.ring_rows(0, 0, 1, h, 0, r.n_kv)
        assert rel_err(ring_k, kr[r.abs_base:, h]) <= 1e-6
        assert np.array_equal(ring_v, v[0, 0, r.abs_base:, h])
    # offline, same kernels
    sb = vrt.offline_scratch_bytes(desc, T)
    scratch = torch.empty(sb, dtype=torch.uint8, device=DEV)
    off = torch.empty_like(qd[0, 0])
    vrt.enc_attn_offline(desc, qd[0, 0], kd[0, 0], vd[0, 0], T, 0, off, scratch, sb, stream())
    off = host(off)
    assert np.array_equal(chunked, off), "chunked != offline"
    ref = attention.windowed(q[0, 0], k[0, 0], v[0, 0], 0, 750, THETA)
    check_close(chunked, ref, vrt.F32, "C0 chunked vs oracle")
    pool.close()


def test_bf16_streams_layers_compactions_any_chunking():
    """2 streams x 2 layers, bf16 N(0,1)*0.5, staggered starts, 1800 frames
    (one compaction per unit) fed in chunks of 4; then of 1, 2, 8 and a mixed
    schedule: every run bit-identical to the 4-frame run."""
    S, L, T, H, d = 2, 2, 1800, 20, 64
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=L)
    starts = offsets(1, S, 0, 750)
    q, k, v = seqs(1, S, L, T, H, d, 0.5, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    pool = Pool(desc, S, starts)
    say("bf16 2x2 units, 4-frame feeds")
    base = host(run_feeds(pool, range(S), 0, L, qd, kd, vd, [4]))
    for s in range(S):
        assert pool.states[s].query(1) == (starts[s] + 786, 1014)
    for s in range(S):
        for l in range(L):
            ref = attention.windowed(q[s, l], k[s, l], v[s, l], int(starts[s]), 750, THETA)
            check_close(base[s, l], ref, vrt.BF16, f"stream {s} layer {l}")
    for sizes in ([1], [2], [8], [3, 5, 1, 7]):
        for s in range(S):
            pool.states[s].reset(int(starts[s]))
        say(f"bf16 chunks {sizes}")
        other = host(run_feeds(pool, range(S), 0, L, qd, kd, vd, sizes))
        assert np.array_equal(other, base), sizes
    pool.close()


def test_batched_equals_serial():
    S, T, H, d = 3, 1600, 20, 64
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=1)
    starts = [5, 400, 123_456]
    q, k, v = seqs(2, S, 1, T, H, d, 0.5, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    say("batched: 3 states in one call")
    pb = Pool(desc, S, starts)
    batched = host(run_feeds(pb, range(S), 0, 1, qd, kd, vd, [4]))
    ps = Pool(desc, S, starts)
    for s in range(S):
        say(f"serial: state {s}")
        one = host(run_feeds(ps, [s], 0, 1, qd[s:s + 1], kd[s:s + 1], vd[s:s + 1], [4]))
        assert np.array_equal(one[0], batched[s])
    pb.close()
    ps.close()


def test_ragged_layers_in_one_call():
    """Layer 1 of state 0 is fed 10 extra frames first, so the layers of that
    state differ in n_kv inside the next calls."""
    L, H, d = 3, 20, 64
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=L)
    pool = Pool(desc, 2, [0, 77])
    T = 900
    q, k, v = seqs(3, 2, L, T + 10, H, d, 0.5, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    say("ragged: layer 1 of state 0 runs 10 frames ahead")
    lead = empty((1, 1, 10, H, d), vrt.BF16)
    vrt.enc_attn_feed([pool.states[0]], 1, 1, qd[0:1, 1:2, :10].contiguous(),
                      kd[0:1, 1:2, :10].contiguous(), vd[0:1, 1:2, :10].contiguous(), 10, lead,
                      stream())
    # afterwards every unit consumes its own sequence: layer 1 of state 0 from
    # frame 10 on, every other unit from frame 0 on
    qs = torch.stack([torch.stack([qd[s, l, (10 if (s, l) == (0, 1) else 0):][:T]
                                   for l in range(L)]) for s in range(2)])
    ks = torch.stack([torch.stack([kd[s, l, (10 if (s, l) == (0, 1) else 0):][:T]
                                   for l in range(L)]) for s in range(2)])
    vs = torch.stack([torch.stack([vd[s, l, (10 if (s, l) == (0, 1) else 0):][:T]
                                   for l in range(L)]) for s in range(2)])
    out = host(run_feeds(pool, [0, 1], 0, L, qs, ks, vs, [4]))
    for s, l in [(0, 0), (0, 1), (1, 2)]:
        o = 10 if (s, l) == (0, 1) else 0
        start = [0, 77][s]
        n = T + o
        ref = attention.windowed_at(q[s, l, :n], k[s, l, :n], v[s, l, :n], start, 750, THETA,
                                    range(n - 40, n))
        check_close(out[s, l, T - 40:], ref, vrt.BF16, f"ragged unit ({s},{l}) last 40")
    pool.close()


def test_large_feed_split_and_offline_fp32():
    """A 1300-frame feed is split 512 + 512 + 276 with a compaction between
    sub-batches; fp32 runs take the VALU path at every size, so it equals
    the offline pass bit for bit."""
    T, H, d = 2600, 20, 64
    desc = vrt.enc_desc(dtype=vrt.F32, n_layers=1)
    q, k, v = seqs(4, 1, 1, T, H, d, 1.0, vrt.F32)
    qd, kd, vd = (to_dev(x, vrt.F32) for x in (q, k, v))
    pool = Pool(desc, 1, [999_000])
    say("fp32 1300-frame feeds")
    big = host(run_feeds(pool, [0], 0, 1, qd, kd, vd, [1300]))[0, 0]
    sb = vrt.offline_scratch_bytes(desc, T)
    scratch = torch.empty(sb, dtype=torch.uint8, device=DEV)
    off = torch.empty_like(qd[0, 0])
    vrt.enc_attn_offline(desc, qd[0, 0], kd[0, 0], vd[0, 0], T, 999_000, off, scratch, sb,
                         stream())
    assert np.array_equal(big, host(off))
    ts = list(range(0, 5)) + list(range(1530, 1545)) + list(range(T - 20, T))
    ref = attention.windowed_at(q[0, 0], k[0, 0], v[0, 0], 999_000, 750, THETA, ts)
    check_close(big[ts], ref, vrt.F32, "1300-frame feeds at positions ~1e6")
    pool.close()


def test_offline_bf16_vs_oracle():
    T, H, d = 700, 20, 64
    desc = vrt.enc_desc(dtype=vrt.BF16)
    q, k, v = qkv(5, 0, 0, T, H, H, d, 0.5, "bf16")
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    sb = vrt.offline_scratch_bytes(desc, T)
    scratch = torch.empty(sb, dtype=torch.uint8, device=DEV)
    out = empty((T, H, d), vrt.BF16)
    say("offline bf16 T=700")
    vrt.enc_attn_offline(desc, qd, kd, vd, T, 31, out, scratch, sb, stream())
    torch.cuda.synchronize()
    ref = attention.windowed(q, k, v, 31, 750, THETA)
    check_close(host(out), ref, vrt.BF16, "offline bf16")


def _dec_run(desc, q, k, v, schedule, n_layers=1):
    """Drive one decoder state through a schedule of n_tok values."""
    T = q.shape[0]
    pool = Pool(desc, 1, [0])
    qd, kd, vd = (to_dev(x, desc.dtype) for x in (q, k, v))
    ws_b = vrt.dec_workspace_bytes(desc, 1, n_layers, 1)
    ws = torch.empty(ws_b // 4 + 1, dtype=torch.float32, device=DEV)
    out = torch.empty_like(qd)
    t = 0
    for n in schedule:
        o = torch.empty_like(qd[t:t + n])
        vrt.dec_attn_step(pool.states, 0, 1, qd[t:t + n].contiguous(), kd[t:t + n].contiguous(),
                          vd[t:t + n].contiguous(), n, o, ws, ws_b, stream())
        out[t:t + n] = o
        t += n
    assert t == T
    torch.cuda.synchronize()
    res = host(out)
    pool.close()
    return res


def test_decoder_ring_equals_linear_and_oracle():
    """GQA 32/8, hd 128, bf16, window 256: a 256-slot modulo ring against a
    1024-slot buffer that never wraps: bit-identical; both vs the oracle."""
    T = 700
    q, k, v = qkv(6, 0, 0, T, 32, 8, 128, 1.0, "bf16")
    sched = [39, 20] + [1] * (T - 59)
    say("decoder window 256: ring 256")
    ring = _dec_run(vrt.dec_desc(window=256, ring_slots=256), q, k, v, sched)
    say("decoder window 256: linear 1024")
    lin = _dec_run(vrt.dec_desc(window=256, ring_slots=1024), q, k, v, sched)
    assert np.array_equal(ring, lin)
    ref = attention.windowed(q, k, v, 0, 256, THETA)
    check_close(ring, ref, vrt.BF16, "decoder ring vs oracle")


def test_decoder_full_window_sampled():
    """Window 8192, ring 8192, past the wrap: 8192 tokens by 512-token
    prefills, then single-token steps to 8300; sampled outputs vs the oracle."""
    T = 8300
    q, k, v = qkv(7, 0, 0, T, 32, 8, 128, 1.0, "bf16")
    sched = [512] * 16 + [1] * (T - 8192)
    say("decoder 8192: prefill 16 x 512 then 108 steps")
    out = _dec_run(vrt.dec_desc(), q, k, v, sched)
    ts = [0, 511, 512, 8191, 8192, 8193, 8250, T - 1]
    ref = attention.windowed_at(q, k, v, 0, 8192, THETA, ts)
    check_close(out[ts], ref, vrt.BF16, "decoder 8192 sampled")
