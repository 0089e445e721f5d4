"""Parity at the launch shapes bench.py times, where the host's launch planner
puts several heads in one workgroup and many units in one launch.

* Decoder step at the shape of the 32-stream x 26-layer serving step: 16
  states x 4 layers of GQA 32/8 x 128, window 8192, every state in one
  vrt_dec_attn_step call per token, with ragged contexts from 39 to 10 269
  tokens (inside the first key split, at the window, past the ring wrap).
  The planner takes 4 kv heads per workgroup and up to 9 key splits there.
  Bar: bit-identical to the same steps made state by state (one kv head per
  workgroup; family doc, Capability Validation table, Batch row: batched
  output byte-identical to serial), the modulo-ring metadata of every state
  as the oracle's ring model gives it, and every state's last output within
  the bf16 bar of the oracle.
* Encoder feed at the shape of the 64-stream x 32-layer staggered workload:
  16 streams x 32 layers (512 units in one launch, 10 heads per workgroup),
  ring phases staggered so that each stream compacts at its own step inside
  the run.  Bar: bit-identical to the same streams fed one at a time (one
  head per workgroup), ring metadata equal to the oracle's ring model, and
  sampled rows (including the first feed after each sampled stream's
  compaction) within the bf16 bar of the oracle.

Inputs are drawn on the GPU from seeded generators; the rows the oracle
checks and the windows they read are copied to the host.  Oracle rows run on
a small thread pool (numpy releases the interpreter lock in its array
arithmetic)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention
from oracle.ring import DecRing, EncRing
from synth import offsets

from gpu_util import DEV, check_close, say, stream

pytestmark = pytest.mark.gpu
THETA = 1.0e6


def randn(gen, shape, scale):
    x = torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32)
    return (x * scale).to(torch.bfloat16)


def as_np(t):
    return t.float().cpu().numpy()


def oracle_rows(jobs):
    """jobs: list of (q, k, v, start, window, t); returns one [Hq][d] row each."""
    def one(j):
        q, k, v, start, window, t = j
        return attention.windowed_at(q, k, v, start, window, THETA, [t])[0]
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        return list(ex.map(one, jobs))


def test_decoder_c4_shape_batched_equals_serial_and_oracle():
    S, L, HQ, HK, DD, WIN = 16, 4, 32, 8, 128, 8192
    ctx = [39, 40, 517, 1023, 1024, 1025, 1500, 2049, 3000, 4100, 6000, 8191, 8192, 8193, 9001,
           10269]
    steps = 3
    T = max(ctx) + steps
    desc = vrt.dec_desc(dtype=vrt.BF16, n_layers=L)
    hg, splits, _ = vrt.attn_plan(desc, S * L, 1)
    say(f"decoder C4 shape: {S} states x {L} layers, contexts {ctx[0]}..{ctx[-1]}, "
        f"planner: {hg} kv heads per workgroup, {splits} splits")
    assert hg > 1 and splits == 5
    assert vrt.attn_plan(desc, L, 1)[0] == 1    # one state alone: one kv head per workgroup
    gen = torch.Generator(device=DEV)
    gen.manual_seed(40)
    q = randn(gen, (S, L, T, HQ, DD), 1.0)
    k = randn(gen, (S, L, T, HK, DD), 1.0)
    v = randn(gen, (S, L, T, HK, DD), 1.0)
    nb = vrt.state_device_bytes(desc)
    pools = []
    for _ in range(2):
        mem = torch.empty(S * nb, dtype=torch.uint8, device=DEV)
        pools.append((mem, [vrt.StreamState(desc, mem[i * nb:(i + 1) * nb], nb, 0) for i in range(S)]))
    wsb = vrt.dec_workspace_bytes(desc, S, L, 1)
    ws = torch.empty(wsb // 4 + 1, dtype=torch.float32, device=DEV)
    st = stream()
    # fill every cache the same way in both pools: a 39-token prefill, prefills
    # of up to 512 tokens up to the window, then single tokens past the wrap
    for i in range(S):
        n = 0
        sched = []
        for m in [39] + [512] * 16:
            m = min(m, min(ctx[i], WIN) - n)
            if m <= 0:
                break
            sched.append(m)
            n += m
        sched += [1] * (ctx[i] - n)
        t = 0
        for m in sched:
            qs, ks, vs = (x[i:i + 1, :, t:t + m].contiguous() for x in (q, k, v))
            o = torch.empty_like(qs)
            for _, states in pools:
                vrt.dec_attn_step([states[i]], 0, L, qs, ks, vs, m, o, ws, wsb, st)
            t += m
    torch.cuda.synchronize()
    say("  caches filled; stepping all states in one call and state by state")
    outs = [torch.empty((steps, S, L, 1, HQ, DD), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    for j in range(steps):
        qs, ks, vs = (torch.stack([x[i, :, ctx[i] + j:ctx[i] + j + 1] for i in range(S)]).contiguous()
                      for x in (q, k, v))
        vrt.dec_attn_step(pools[0][1], 0, L, qs, ks, vs, 1, outs[0][j], ws, wsb, st)
        for i in range(S):
            o = torch.empty_like(qs[i:i + 1])
            vrt.dec_attn_step([pools[1][1][i]], 0, L, qs[i:i + 1].contiguous(), ks[i:i + 1].contiguous(),
                              vs[i:i + 1].contiguous(), 1, o, ws, wsb, st)
            outs[1][j, i] = o[0]
    torch.cuda.synchronize()
    a, b = as_np(outs[0]), as_np(outs[1])
    assert np.isfinite(a).all()
    assert np.array_equal(a, b), "batched decoder step != state by state"
    for i in range(S):
        r = DecRing(WIN)
        r.reset(0)
        r.append(ctx[i] + steps)
        for pool in pools:
            for l in (0, L - 1):
                assert pool[1][i].query(l) == (0, r.next_pos), (i, l)
    # every state's last output against the oracle (layer i % L)
    jobs = []
    for i in range(S):
        l, t = i % L, ctx[i] + steps - 1
        lo = max(0, t - WIN + 1)
        jobs.append((as_np(q[i, l, lo:t + 1]), as_np(k[i, l, lo:t + 1]), as_np(v[i, l, lo:t + 1]),
                     lo, WIN, t - lo))
    say(f"  oracle: {S} rows of windows up to {WIN} keys")
    refs = oracle_rows(jobs)
    for i in range(S):
        check_close(a[steps - 1, i, i % L, 0], refs[i], vrt.BF16, f"state {i} ctx {ctx[i]}")
    for _, states in pools:
        for s in states:
            s.close()


def test_encoder_c1_shape_batched_equals_one_stream_at_a_time():
    S, L, H, D, W, n, steps = 16, 32, 20, 64, 750, 4, 40
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=L)
    hg, _, _ = vrt.attn_plan(desc, S * L, n)
    say(f"encoder C1 shape: {S} streams x {L} layers = {S * L} units, {hg} heads per workgroup")
    assert hg == 10
    assert vrt.attn_plan(desc, L, n)[0] == 1
    # rows held before the 4-frame feeds: each stream compacts once, at its
    # own step, inside the run
    pre = [int(x) for x in offsets(41, S, 1376, 1533)]
    starts = [int(x) for x in offsets(42, S, 0, 10 ** 6)]
    T = max(pre) + steps * n
    gen = torch.Generator(device=DEV)
    gen.manual_seed(41)
    q, k, v = (randn(gen, (S, L, T, H, D), 0.5) for _ in range(3))
    nb = vrt.state_device_bytes(desc)
    pools = []
    for _ in range(2):
        mem = torch.empty(S * nb, dtype=torch.uint8, device=DEV)
        pools.append((mem, [vrt.StreamState(desc, mem[j * nb:(j + 1) * nb], nb, starts[j])
                            for j in range(S)]))
    st = stream()
    for i in range(S):
        qs, ks, vs = (x[i:i + 1, :, :pre[i]].contiguous() for x in (q, k, v))
        o = torch.empty_like(qs)
        for _, states in pools:
            vrt.enc_attn_feed([states[i]], 0, L, qs, ks, vs, pre[i], o, st)
    torch.cuda.synchronize()
    say("  rings filled; feeding all streams in one call and one stream at a time")
    outs = [torch.empty((steps, S, L, n, H, D), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    for j in range(steps):
        qs, ks, vs = (torch.stack([x[i, :, pre[i] + n * j:pre[i] + n * (j + 1)] for i in range(S)]).contiguous()
                      for x in (q, k, v))
        vrt.enc_attn_feed(pools[0][1], 0, L, qs, ks, vs, n, outs[0][j], st)
        for i in range(S):
            o = torch.empty_like(qs[i:i + 1])
            vrt.enc_attn_feed([pools[1][1][i]], 0, L, qs[i:i + 1].contiguous(), ks[i:i + 1].contiguous(),
                              vs[i:i + 1].contiguous(), n, o, st)
            outs[1][j, i] = o[0]
    torch.cuda.synchronize()
    a, b = as_np(outs[0]), as_np(outs[1])
    assert np.isfinite(a).all()
    assert np.array_equal(a, b), "512-unit launch != one stream at a time"
    comp_step = []
    for i in range(S):
        r = EncRing()
        r.reset(starts[i])
        r.feed(pre[i])
        first = None
        for j in range(steps):
            before = len(r.events)
            r.feed(n)
            if first is None and len(r.events) > before:
                first = j
        assert first is not None, i
        comp_step.append(first)
        for pool in pools:
            for l in (0, 17, L - 1):
                assert pool[1][i].query(l) == (r.abs_base, r.n_kv), (i, l)
    say(f"  compaction steps per stream: {comp_step}")
    assert len(set(comp_step)) > 4
    rng = np.random.default_rng(43)
    jobs, where = [], []
    for i in (0, 5, 9, 15):
        for l in (i % L, (i * 7 + 3) % L):
            for j in sorted({comp_step[i], steps - 1, int(rng.integers(0, steps))}):
                for f in (0, n - 1):
                    t = pre[i] + n * j + f
                    lo = max(0, t - W + 1)
                    jobs.append((as_np(q[i, l, lo:t + 1]), as_np(k[i, l, lo:t + 1]),
                                 as_np(v[i, l, lo:t + 1]), starts[i] + lo, W, t - lo))
                    where.append((i, l, j, f))
    say(f"  oracle: {len(jobs)} sampled rows")
    refs = oracle_rows(jobs)
    got = np.stack([a[j, i, l, f] for i, l, j, f in where])
    check_close(got, np.stack(refs), vrt.BF16, "C1-shape sampled rows")
    for _, states in pools:
        for s in states:
            s.close()


@pytest.mark.parametrize("dtype, n, S, hg_expect", [(vrt.F32, 8, 16, 2), (vrt.BF16, 16, 16, 2),
                                                   (vrt.BF16, 8, 32, 5)])
def test_encoder_multirow_feeds_batched_equals_one_stream_at_a_time(dtype, n, S, hg_expect):
    """Vector-path feeds of 8 or 16 frames (8 or 16 query rows per head, four
    per wave) across S streams x 8 layers, where the planner takes several kv
    heads per workgroup: equal bit for bit to each stream fed alone (one head
    per workgroup), across each stream's compaction; sampled rows against the
    oracle."""
    L, H, D, W, steps = 8, 20, 64, 750, 8
    tdt = torch.bfloat16 if dtype == vrt.BF16 else torch.float32
    desc = vrt.enc_desc(dtype=dtype, n_layers=L)
    hg, _, _ = vrt.attn_plan(desc, S * L, n)
    say(f"multi-row feeds: {n} frames, {S} streams x {L} layers, {hg} heads per workgroup")
    assert hg == hg_expect and vrt.attn_plan(desc, L, n)[0] == 1
    pre = [int(x) for x in offsets(61, S, 1536 - steps * n + 1, 1530)]   # each ring compacts inside the run
    starts = [int(x) for x in offsets(62, S, 0, 10 ** 6)]
    T = max(pre) + steps * n
    gen = torch.Generator(device=DEV)
    gen.manual_seed(61 + n + S)
    q, k, v = ((torch.randn((S, L, T, H, D), generator=gen, device=DEV) * 0.5).to(tdt) for _ in range(3))
    nb = vrt.state_device_bytes(desc)
    pools = []
    for _ in range(2):
        mem = torch.empty(S * nb, dtype=torch.uint8, device=DEV)
        pools.append((mem, [vrt.StreamState(desc, mem[j * nb:(j + 1) * nb], nb, starts[j]) for j in range(S)]))
    st = stream()
    for i in range(S):
        qs, ks, vs = (x[i:i + 1, :, :pre[i]].contiguous() for x in (q, k, v))
        o = torch.empty_like(qs)
        for _, states in pools:
            vrt.enc_attn_feed([states[i]], 0, L, qs, ks, vs, pre[i], o, st)
    outs = [torch.empty((steps, S, L, n, H, D), dtype=tdt, device=DEV) for _ in range(2)]
    for j in range(steps):
        qs, ks, vs = (torch.stack([x[i, :, pre[i] + n * j:pre[i] + n * (j + 1)] for i in range(S)]).contiguous()
                      for x in (q, k, v))
        vrt.enc_attn_feed(pools[0][1], 0, L, qs, ks, vs, n, outs[0][j], st)
        for i in range(S):
            o = torch.empty_like(qs[i:i + 1])
            vrt.enc_attn_feed([pools[1][1][i]], 0, L, qs[i:i + 1].contiguous(), ks[i:i + 1].contiguous(),
                              vs[i:i + 1].contiguous(), n, o, st)
            outs[1][j, i] = o[0]
    torch.cuda.synchronize()
    a, b = as_np(outs[0]), as_np(outs[1])
    assert np.isfinite(a).all()
    assert np.array_equal(a, b), "batched launch != one stream at a time"
    for i in range(S):
        r = EncRing()
        r.reset(starts[i])
        r.feed(pre[i])
        for _ in range(steps):
            r.feed(n)
        assert r.events, ("no compaction", i)
        for pool in pools:
            assert pool[1][i].query(L - 1) == (r.abs_base, r.n_kv), i
    jobs, where = [], []
    for i in (0, S // 2, S - 1):
        for l in (0, L - 1):
            for j, f in ((0, 0), (steps - 1, n - 1)):
                t = pre[i] + n * j + f
                lo = max(0, t - W + 1)
                jobs.append((as_np(q[i, l, lo:t + 1]), as_np(k[i, l, lo:t + 1]), as_np(v[i, l, lo:t + 1]),
                             starts[i] + lo, W, t - lo))
                where.append((i, l, j, f))
    refs = oracle_rows(jobs)
    got = np.stack([a[j, i, l, f] for i, l, j, f in where])
    check_close(got, np.stack(refs), dtype, f"multi-row feeds {n} frames, sampled rows")
    for _, states in pools:
        for s in states:
            s.close()
