#!/usr/bin/env python3
"""Throughput of streamed windowed-750 encoder attention on one MI355X.

Configurations (--config):

c2 (default)  steady-state serving: 256 independent streams x 1 layer, 20
              heads x 64, window 750, 1536-slot rings pre-filled to 750 frames
              (untimed), bf16 inputs N(0,1)*0.5 drawn on the GPU from a seeded
              generator, absolute start positions uniform in [1e4, 1e6).  One
              step = one feed call that pushes 4 new frames into every stream:
              ring compaction where due, RoPE + append, windowed attention
              (one fused launch on the vector path).
c1            64 streams x 32 layers, staggered ring phases, 4 frames per step
c3            catch-up: 1 stream x 32 layers, bf16 N(0,1), 15300 frames fed as
              29 batches of 512 + one of 452 (the maximum batch), compactions
              before batches 4..30.  One step = one batch through all 32
              layers: compaction, RoPE + append, attention on the matrix
              cores.  The sequence restarts (host-only reset) after its last
              batch.
c2b           the c2 step through the attention half of an encoder block
              (RMSNorm, q/k/v projection, the path, output projection).
c4            decoder step: 32 streams x 26 layers, GQA 32/8 x 128, window 8192.
cs            the causal conv stem: 256 streams x 8 mel frames per step.
cm            six (left, right)-window layers without RoPE (the moonshine pattern).
copy          calibration copy of 1 GiB for the HBM byte counters.
read          calibration: a plain streaming read of 4 GiB (the practical ceiling).
stream        calibration: the serving step's tile stream with no arithmetic, and its L2 rate per CU.
gemm          calibration: the block's two projections at the serving shape, the library's
              GEMM against the vendor BLAS (torch.matmul), each replayed from a HIP graph.

--ring mod runs c1, c2 or c3 with the encoder cache kept as a modulo ring
(1280 slots, slot = position % slots, no compaction; outputs bit-identical
to the compacting ring).

All inputs of all timed steps are resident in HBM before the timed region.
Prints one JSON line: frames/s over all streams (a frame counts once, after
every layer of the configuration has processed it), the roofline of the
attention kernel (algorithmic bytes or flops per launch / its per-launch time
from HIP events recorded on the launch stream) and the fp64 CPU oracle timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak, published
H, D, W = 20, 64, 750
R = H * D
METRIC = "encoder frames/s through cached window-750 attention (all streams); % HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_work(n_kv: int, n: int, elem: int = 2):
    """Algorithmic bytes and flops of one unit-step of the path (RoPE, append
    and attention) over a sub-batch of n frames when the ring held n_kv rows
    before it, in its fused minimum: read the n new q, k and v rows, write the
    n rotated-key and value rows into the ring, read the keys and values of
    the min(n_kv, W-1) older rows of the window, write n outputs:
    (3n + 2n + 2 old + n) R e bytes; 4 d flops per (query, visible key) per
    head."""
    old = min(n_kv, W - 1)
    nbytes = (6 * n + 2 * old) * R * elem
    visible = sum(min(W, n_kv + j + 1) for j in range(n))
    return nbytes, 4 * D * H * visible


def attn_kernel_bytes(n_kv: int, n: int, elem: int = 2) -> int:
    """Bytes the matrix-path attention kernel itself must move for one unit
    (its rows were appended by a separate launch): the n queries, the keys
    and values of the whole window (old rows and the n new ones), n outputs."""
    old = min(n_kv, W - 1)
    return (n + 2 * (old + n) + n) * R * elem


def compaction_bytes(units: int, elem: int = 2) -> int:
    """One compaction per unit: the last W rows of K and V read and written."""
    return units * 2 * 2 * W * R * elem


def oracle_stream_run(job):
    """One single-layer stream of the fp64 oracle (streamed form): pre-filled
    with `pre` frames (not timed), then `steps` feeds of `n` frames, timed.
    Returns (start, end) of the timed feeds on the system-wide monotonic
    clock.  Runs in the calling process on one BLAS thread."""
    from threadpoolctl import threadpool_limits
    from oracle.stream import EncStream
    from synth import qkv

    seed, s, start, pre, steps, n, scale = job
    with threadpool_limits(limits=1):
        T = pre + steps * n
        q, k, v = qkv(seed, s, 0, T, H, H, D, scale, "bf16")
        st = EncStream(H, D, start_pos=int(start))
        if pre:
            st.feed(q[:pre], k[:pre], v[:pre])
        t0 = time.perf_counter()
        for i in range(steps):
            a = pre + i * n
            st.feed(q[a:a + n], k[a:a + n], v[a:a + n])
        return t0, time.perf_counter()


CPU_POOL = None


def start_cpu_pool():
    """Worker processes for the all-core oracle baseline, started before
    anything touches the GPU (each is a fresh interpreter; nothing is forked
    from a process that holds the GPU).  One per host core of this job's
    share, at most 16."""
    global CPU_POOL
    import multiprocessing as mp
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    CPU_POOL = (mp.get_context("spawn").Pool(n), n)


def cpu_baseline(layers_in_config: int, pre: int, steps: int, n: int, scale: float, starts, what: str,
                 seed: int, steps_1t: int = None):
    """The fp64 oracle (streamed form, the method itself) on a bounded sample
    of the workload: single-layer streams pre-filled with `pre` frames (not
    timed), then `steps` feeds of `n` frames (timed).  All cores: one stream
    per worker process, all at once, the rate taken over the span from the
    first worker's start to the last one's end.  One thread: one stream in
    this process.  Rates are divided by the configuration's layer count, so
    they are in the same unit as the GPU value (frames through every layer)."""
    steps_1t = steps if steps_1t is None else steps_1t
    t0, t1 = oracle_stream_run((seed, 0, int(starts[0]), pre, steps_1t, n, scale))
    one = {"value": steps_1t * n / (t1 - t0) / layers_in_config, "threads": 1,
           "sample": f"1 stream x 1 layer x {steps_1t} feeds of {n} frames, {t1 - t0:.1f} s"}
    res = {"value": one["value"], "unit": "frames/s", "cores": 1, "kind": "oracle",
           "host_cpu_count": os.cpu_count(), "single_thread": one}
    if CPU_POOL is not None:
        pool, nproc = CPU_POOL
        jobs = [(seed, s, int(starts[s % len(starts)]), pre, steps, n, scale) for s in range(nproc)]
        spans = pool.map_async(oracle_stream_run, jobs).get(timeout=600)
        span = max(b for _, b in spans) - min(a for a, _ in spans)
        res["value"] = nproc * steps * n / span / layers_in_config
        res["cores"] = nproc
        res["sample"] = (f"{what}: {nproc} streams x 1 layer x {steps} feeds of {n} frames, one stream "
                         f"per worker process on {nproc} host cores at once (rings pre-filled with {pre} "
                         f"frames, not timed), oracle.stream.EncStream in fp64 numpy, one BLAS thread "
                         f"each, {span:.1f} s from the first start to the last end for {nproc * steps * n} "
                         f"frame-layers, divided by {layers_in_config} layer(s) per frame; "
                         f"single_thread: the same on one stream in one thread")
    else:
        res["sample"] = (f"{what}: " + one["sample"] + f" (rings pre-filled with {pre} frames, not timed), "
                         f"oracle.stream.EncStream in fp64 numpy on one thread, divided by "
                         f"{layers_in_config} layer(s) per frame")
    return res


def cpu_baseline_block(steps: int):
    """The fp64 oracle through the attention half of a block, streamed: one
    stream, rings pre-filled with 750 frames (not timed), then `steps` feeds
    of 4 frames (timed): RMSNorm and projections (oracle.block) around
    oracle.stream.EncStream."""
    import numpy as np
    from oracle import block
    from oracle.stream import EncStream
    from synth import block_input, block_weights

    dim = H * D
    wts = block_weights(5, 0, dim)
    T = W + 4 * steps
    x = block_input(5, 0, 0, T, dim)
    st = EncStream(H, D, start_pos=12345)

    def feed(xc):
        y = block.rmsnorm(xc, wts["norm_w"])
        q = block.linear(y, wts["wq"], wts["bq"]).reshape(-1, H, D)
        k = block.linear(y, wts["wk"]).reshape(-1, H, D)
        v = block.linear(y, wts["wv"], wts["bv"]).reshape(-1, H, D)
        a = np.asarray(st.feed(q, k, v)).reshape(-1, dim)
        return xc + block.linear(a, wts["wo"], wts["bo"])

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):   # one host thread, like the other oracle baselines
        feed(x[:W])
        t0 = time.perf_counter()
        for i in range(steps):
            feed(x[W + 4 * i:W + 4 * i + 4])
        el = time.perf_counter() - t0
    return {"value": 4 * steps / el, "unit": "frames/s", "cores": 1, "kind": "oracle",
            "sample": f"one stream x 1 layer, {steps} feeds of 4 frames through the block's attention "
                      f"half (rings pre-filled with 750 frames, not timed), oracle.block + "
                      f"oracle.stream.EncStream in fp64 numpy, {el:.1f} s"}


def cpu_baseline_dec(contexts, steps: int = 80):
    """The fp64 oracle's decoder stream (oracle.stream.DecStream) on a bounded
    sample: one layer of one stream at the median context, `steps` timed
    single-token steps after an untimed fill; scaled to tokens/s through 26
    layers."""
    import numpy as np
    from oracle import rope
    from oracle.stream import DecStream
    from synth import qkv

    c = sorted(contexts)[len(contexts) // 2]
    q, k, v = qkv(4, 0, 0, c + steps, 32, 8, 128, 1.0, "bf16")
    st = DecStream(32, 8, 128)
    # untimed fill of the oracle's ring (its own RoPE and ring model; no
    # attention outputs are needed for the tokens before the timed steps)
    kr = rope.apply(np.asarray(k[:c], dtype=np.float64), np.arange(c, dtype=np.int64), 1.0e6)
    for p, slot in st.ring.append(c):
        st.K[slot] = kr[p]
        st.V[slot] = v[p]
    t0 = time.perf_counter()
    for j in range(steps):
        st.step(q[c + j:c + j + 1], k[c + j:c + j + 1], v[c + j:c + j + 1])
    el = time.perf_counter() - t0
    return {"value": steps / el / 26, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"one decoder layer of one stream at context {c} (the median), {steps} timed "
                      f"single-token steps after an untimed ring fill, oracle.stream.DecStream in fp64 "
                      f"numpy on one thread, {el:.1f} s; divided by 26 layers per token"}


def _randn(gen, shape, scale, dev):
    import torch
    x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    return (x * scale).to(torch.bfloat16)


def enc_desc(args, layers):
    import sliding_window_cached_amd as vrt
    kind = vrt.ENC_MODRING if args.ring == "mod" else vrt.ENC_RING
    return vrt.enc_desc(dtype=vrt.BF16, n_layers=layers, kind=kind)


def ring_words(desc) -> str:
    if desc.kind == 0:
        return f"{desc.ring_slots}-slot ring compacted to its last 750 frames when full"
    return f"{desc.ring_slots}-slot modulo ring (slot = position % {desc.ring_slots}, no compaction)"


DEVICE_WARMUP_S = 0.5


def device_warmup(seconds: float = None):
    """Bring the GPU to its sustained clocks before the warmup steps: for
    `seconds` of wall time, untimed, alternate the library's read probe over a
    1 GiB buffer with bf16 8192 x 8192 products (torch.matmul).  On a freshly
    leased MI355X the first attention launches run slower than the steady
    state; on one machine, 20 serving steps after 5 warmup steps took 175.9 and
    178.3 us per launch (median) after a read-only warm-up, 171.3 and 171.9 us
    after this mixed one, 171.9 us after 200 warmup steps instead, and 173.6 us
    over 1000 steps.  A streaming read alone leaves the core clock low.  No
    state of the workload is touched, and nothing of it is timed."""
    import torch
    import sliding_window_cached_amd as vrt
    seconds = DEVICE_WARMUP_S if seconds is None else seconds
    if seconds <= 0:
        return
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(0)
    a = torch.randn(8192, 8192, generator=gen, device="cuda:0").to(torch.bfloat16)
    b = torch.randn(8192, 8192, generator=gen, device="cuda:0").to(torch.bfloat16)
    stream = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            vrt.read_probe(buf, buf.numel(), sink, stream)
        for _ in range(8):
            torch.matmul(a, b)
        torch.cuda.synchronize()
    del buf, sink, a, b


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it
    skips the system-scope release fence (cache writeback and invalidation) a
    default event performs, so bracketing every launch of a short run with
    events does not slow the launches in between (measured on the serving
    step: 182 us of wall time per step with default events around every
    launch, 174 us with them around every tenth; the kernel durations are the
    same).  The events only measure time.  Recorded on torch's current
    stream; `cuda_event` is the raw hipEvent_t for vrt.set_attn_events."""
    _hip = None
    FLAGS = 0x20000000   # hipEventDisableSystemFence

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            import sliding_window_cached_amd as vrt
            lib = ctypes.CDLL(vrt.HIP_RUNTIME or "libamdhip64.so")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        h = ctypes.c_void_p()
        if self.hip().hipEventCreateWithFlags(ctypes.byref(h), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = h.value

    def record(self):
        import torch
        if self.hip().hipEventRecord(self.cuda_event, torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        if self.hip().hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        try:
            if self.cuda_event:
                self.hip().hipEventDestroy(self.cuda_event)
        except Exception:
            pass


def _timing_events(n):
    import torch
    evs = [(TimingEvent(), TimingEvent()) for _ in range(n)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    return evs


def bench_c2(args):
    import torch
    import sliding_window_cached_amd as vrt
    from synth import offsets

    dev = torch.device("cuda:0")
    S, n = 256, 4
    desc = enc_desc(args, 1)
    starts = offsets(2, S, 10 ** 4, 10 ** 6)
    nb = vrt.state_device_bytes(desc)
    mem = torch.empty(S * nb, dtype=torch.uint8, device=dev)
    states = [vrt.StreamState(desc, mem[i * nb:(i + 1) * nb], nb, int(starts[i])) for i in range(S)]
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)

    log("c2: pre-filling 256 rings to 750 frames")
    pre = [_randn(gen, (S, 1, W, H, D), 0.5, dev) for _ in range(3)]
    pre_out = torch.empty_like(pre[0])
    vrt.enc_attn_feed(states, 0, 1, pre[0], pre[1], pre[2], W, pre_out, stream)
    torch.cuda.synchronize()
    del pre, pre_out
    total = args.warmup + args.steps
    log(f"c2: drawing inputs for {total} steps into HBM")
    Q, K, V = (_randn(gen, (total, S, 1, n, H, D), 0.5, dev) for _ in range(3))
    out = torch.empty((S, 1, n, H, D), dtype=torch.bfloat16, device=dev)

    # which timed steps compact (all rings share one schedule here) and the
    # ring occupancy each step's attention sees, from the ring model; and the
    # timing events.  Worked out before the warmup steps, so that nothing
    # leaves the GPU idle between them and the timed steps.
    _, nkv = states[0].query(0)
    for i in range(args.warmup):
        _, nkv, _ = vrt.ring_advance(desc, 0, nkv, n)
    compacting, nkv_seen = [], []
    for i in range(args.steps):
        _, nkv_after, nc = vrt.ring_advance(desc, 0, nkv, n)
        compacting.append(nc > 0)
        nkv_seen.append(nkv_after - n)
        nkv = nkv_after
    every = max(1, args.timing_every or (1 if args.steps < 100 else 10))
    timed = list(range(0, args.steps, every))
    ev = dict(zip(timed, _timing_events(len(timed))))

    device_warmup()
    for i in range(args.warmup):
        vrt.enc_attn_feed(states, 0, 1, Q[i], K[i], V[i], n, out, stream)
    log(f"c2: timing {args.steps} steps (attention events on every {every})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        i = args.warmup + j
        if j in ev:
            vrt.set_attn_events(ev[j][0], ev[j][1])
        elif every > 1 and j - 1 in ev:
            vrt.set_attn_events()
        vrt.enc_attn_feed(states, 0, 1, Q[i], K[i], V[i], n, out, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    vrt.set_attn_events()
    attn_ms = [ev[j][0].elapsed_time(ev[j][1]) for j in timed]
    srt = sorted(attn_ms)
    log(f"c2: attention launches (us): min {srt[0] * 1e3:.1f}, median {srt[len(srt) // 2] * 1e3:.1f}, "
        f"max {srt[-1] * 1e3:.1f}; first {attn_ms[0] * 1e3:.1f}")

    # one compaction of all 256 rings (every 196 steps in steady state: the
    # ring goes from 754 to 1536 rows 4 at a time), timed on its own after
    # the timed steps, with events on the launch stream
    comp_every = (desc.ring_slots - W) // n if desc.kind == vrt.ENC_RING else None
    comp = None
    if comp_every:
        cev = _timing_events(3)
        comp_ms = []
        for a, b in cev:
            vrt.enc_attn_feed(states, 0, 1, Q[-1], K[-1], V[-1], n, out, stream)   # n_kv > W again
            a.record()
            vrt.ring_compact(states, 0, 1, stream)
            b.record()
        torch.cuda.synchronize()
        comp_ms = sorted(a.elapsed_time(b) for a, b in cev)
        cb = compaction_bytes(S)
        c_us = comp_ms[1] * 1e3
        comp = {"launch_us": c_us, "bytes": cb, "achieved_gbs": cb / (c_us * 1e-6) / 1e9,
                "every_steps": comp_every,
                "note": "k_compact over all 256 rings, median of 3 launches timed with events after "
                        "the timed steps; in steady state one step in every_steps carries it"}
    for s in states:
        s.close()

    frames = args.steps * S * n
    nbytes = [S * attn_work(nkv_seen[j], n)[0] for j in timed]   # the sampled launches
    t_kernel = sum(attn_ms) * 1e-3 / len(attn_ms)
    achieved = sum(nbytes) / (sum(attn_ms) * 1e-3) / 1e9
    if comp:
        step_s = wall / args.steps
        comp["value_amortized"] = S * n / (step_s + comp["launch_us"] * 1e-6 / comp_every)
        comp["roofline_frac_amortized"] = (
            (nbytes[-1] + comp["bytes"] / comp_every) / (t_kernel + comp["launch_us"] * 1e-6 / comp_every)
            / 1e9 / HBM_PEAK_GBS)
    return {
        "metric": METRIC,
        "value": frames / wall,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "steady-state serving: 256 streams x 1 layer, 20 heads x 64, window 750, "
                        f"{ring_words(desc)}, pre-filled to 750 frames, 4 frames per stream per step, bf16 "
                        "N(0,1)*0.5, start positions U[1e4, 1e6)",
            "streams": S, "layers": 1, "frames_per_step": n, "heads": H, "head_dim": D,
            "window": W, "ring_slots": desc.ring_slots, "ring": args.ring,
            "parallelism": "none (1 GPU)", "device_warmup_s": DEVICE_WARMUP_S,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_attn (vector path: fused RoPE + append + attention, one launch per step)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": (measured_traffic("k_attn", workload_key(args, "c2")) or {}).get("bytes"),
            "alg_bytes_per_launch": nbytes[-1],
            "bytes_model": "(3n + 2n + 2 old + n) * 1280 * 2 B per stream: n = 4 new q, k, v rows "
                           "read, their K/V rows written, old = 749 window rows of K and V read, n "
                           "outputs written",
            "launch_us_mean": t_kernel * 1e6,
            "launches_timed": len(attn_ms),
        },
        "compaction_steps": sum(compacting),
        "compaction": comp,
        "step_hbm_frac": sum(S * attn_work(k, n)[0] for k in nkv_seen) / wall / 1e9 / HBM_PEAK_GBS,
    }


def bench_c2b(args):
    """The serving step of c2 through the whole attention half of an encoder
    block: RMSNorm, the q/k/v projection (one GEMM, 1280 -> 3840, q and v
    biases), the cached path, the output projection with bias and the
    residual.  Random weights: gain 1 + 0.1 N(0,1), matrices N(0, 1/1280),
    biases 0.1 N(0,1); inputs x ~ N(0,1); all bf16."""
    import torch
    import sliding_window_cached_amd as vrt
    from synth import offsets

    dev = torch.device("cuda:0")
    S, n, dim = 256, 4, H * D
    desc = enc_desc(args, 1)
    starts = offsets(2, S, 10 ** 4, 10 ** 6)
    nb = vrt.state_device_bytes(desc)
    mem = torch.empty(S * nb, dtype=torch.uint8, device=dev)
    states = [vrt.StreamState(desc, mem[i * nb:(i + 1) * nb], nb, int(starts[i])) for i in range(S)]
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    norm_w = (1.0 + 0.1 * torch.randn(dim, generator=gen, device=dev)).to(torch.bfloat16)
    w_qkv = _randn(gen, (3 * dim, dim), dim ** -0.5, dev)
    w_o = _randn(gen, (dim, dim), dim ** -0.5, dev)
    b_q, b_v, b_o = (_randn(gen, (dim,), 0.1, dev) for _ in range(3))
    bw = vrt.block_weights(norm_w, w_qkv, b_q, b_v, w_o, b_o, 1.0e-5)

    log("c2b: pre-filling 256 rings to 750 frames through the block")
    xp = _randn(gen, (S, W, dim), 1.0, dev)
    wsb = vrt.block_workspace_bytes(desc, S * W)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    vrt.enc_block_feed(states, 0, xp, W, bw, torch.empty_like(xp), ws, wsb, stream)
    torch.cuda.synchronize()
    del xp, ws
    total = args.warmup + args.steps
    X = _randn(gen, (total, S, n, dim), 1.0, dev)
    out = torch.empty((S, n, dim), dtype=torch.bfloat16, device=dev)
    wsb = vrt.block_workspace_bytes(desc, S * n)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    device_warmup()
    for i in range(args.warmup):
        vrt.enc_block_feed(states, 0, X[i], n, bw, out, ws, wsb, stream)
    torch.cuda.synchronize()
    _, nkv = states[0].query(0)
    nkv_seen = []
    for i in range(args.steps):
        _, nkv_after, _ = vrt.ring_advance(desc, 0, nkv, n)
        nkv_seen.append(nkv_after - n)
        nkv = nkv_after

    every = max(1, args.timing_every or (1 if args.steps < 100 else 10))
    timed = list(range(0, args.steps, every))
    ev = dict(zip(timed, _timing_events(len(timed))))
    blk = dict(zip(timed, _timing_events(len(timed))))
    log(f"c2b: timing {args.steps} block steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        if j in ev:
            vrt.set_attn_events(ev[j][0], ev[j][1])
            blk[j][0].record()
        elif every > 1 and j - 1 in ev:
            vrt.set_attn_events()
        vrt.enc_block_feed(states, 0, X[args.warmup + j], n, bw, out, ws, wsb, stream)
        if j in blk:
            blk[j][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    vrt.set_attn_events()
    attn_ms = [ev[j][0].elapsed_time(ev[j][1]) for j in timed]
    blk_ms = [blk[j][0].elapsed_time(blk[j][1]) for j in timed]
    for st in states:
        st.close()
    M = S * n
    proj_flops = 2 * M * dim * (3 * dim) + 2 * M * dim * dim
    nbytes = [S * attn_work(nkv_seen[j], n)[0] for j in timed]
    t_attn = sum(attn_ms) * 1e-3 / len(attn_ms)
    t_blk = sum(blk_ms) * 1e-3 / len(blk_ms)
    achieved = sum(nbytes) / (sum(attn_ms) * 1e-3) / 1e9
    return {
        "metric": "encoder frames/s through the attention half of a block (norm, projections, "
                  "cached window-750 attention, output projection; all streams)",
        "value": S * n * args.steps / wall,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (random weights)",
        "config": {
            "workload": f"serving step through the attention half of an encoder block: 256 streams x "
                        f"1 layer, d_model 1280 = 20 heads x 64, window 750, {ring_words(desc)}, "
                        "pre-filled to 750 frames, 4 frames per stream per step, x ~ N(0,1), "
                        "random weights, bf16",
            "streams": S, "layers": 1, "frames_per_step": n, "d_model": dim, "window": W,
            "ring_slots": desc.ring_slots, "ring": args.ring, "parallelism": "none (1 GPU)", "device_warmup_s": DEVICE_WARMUP_S,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_attn (the cached path inside the block)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": (measured_traffic("k_attn", workload_key(args, "c2b")) or {}).get("bytes"),
            "launch_us_mean": t_attn * 1e6,
            "launches_timed": len(attn_ms),
        },
        "block": {
            "us_mean": t_blk * 1e6,
            "attention_us_mean": t_attn * 1e6,
            "norm_and_projections_us_mean": (t_blk - t_attn) * 1e6,
            "projection_flops_per_step": proj_flops,
            "projection_tflops_incl_norm": proj_flops / (t_blk - t_attn) / 1e12,
        },
    }


def bench_cs(args):
    """The conv stem at the serving shape: 256 streams, 8 new mel frames per
    stream per step (the pages' chunk), 128 mel bins -> 1280, giving 4
    encoder frames per stream per step.  Random weights N(0, 1/fan_in),
    biases 0.1 N(0,1), mel ~ N(0,1); bf16."""
    import torch
    import sliding_window_cached_amd as vrt

    dev = torch.device("cuda:0")
    S, n, n_mel, d = 256, 8, 128, H * D
    nb = vrt.conv_stem_device_bytes(n_mel, d)
    mem = torch.empty(S * nb, dtype=torch.uint8, device=dev)
    stems = [vrt.ConvStem(n_mel, d, mem[i * nb:(i + 1) * nb], nb) for i in range(S)]
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    w0 = _randn(gen, (d, 3 * n_mel), (3 * n_mel) ** -0.5, dev)
    w1 = _randn(gen, (d, 3 * d), (3 * d) ** -0.5, dev)
    b0, b1 = (_randn(gen, (d,), 0.1, dev) for _ in range(2))
    cw = vrt.conv_weights(w0, b0, w1, b1)
    total = args.warmup + args.steps
    mel = _randn(gen, (total, S, n, n_mel), 1.0, dev)
    out = torch.empty((S, n // 2, d), dtype=torch.bfloat16, device=dev)
    wsb = vrt.conv_workspace_bytes(n_mel, d, S, n)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    device_warmup()
    for i in range(args.warmup):
        vrt.conv_stem_feed(stems, mel[i], n, cw, out, ws, wsb, stream)
    torch.cuda.synchronize()
    every = max(1, args.timing_every or (1 if args.steps < 100 else 10))
    timed = list(range(0, args.steps, every))
    ev = dict(zip(timed, _timing_events(len(timed))))
    log(f"cs: timing {args.steps} conv stem steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        if j in ev:
            ev[j][0].record()
        vrt.conv_stem_feed(stems, mel[args.warmup + j], n, cw, out, ws, wsb, stream)
        if j in ev:
            ev[j][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [ev[j][0].elapsed_time(ev[j][1]) for j in timed]
    for st in stems:
        st.close()
    t_step = sum(ms) * 1e-3 / len(ms)
    flops = 2 * S * n * d * 3 * n_mel + 2 * S * (n // 2) * d * 3 * d
    tfs = flops / t_step / 1e12
    return {
        "metric": "encoder frames/s out of the causal conv stem (all streams)",
        "value": S * (n // 2) * args.steps / wall,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (random weights)",
        "config": {
            "workload": "conv stem serving step: 256 streams, 8 new mel frames each (128 bins), conv "
                        "128 -> 1280 k3 s1 and 1280 -> 1280 k3 s2 with bias and GELU, padding caches; "
                        "4 encoder frames per stream per step",
            "streams": S, "mel_frames_per_step": n, "n_mel": n_mel, "d_model": d,
            "parallelism": "none (1 GPU)", "device_warmup_s": DEVICE_WARMUP_S,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "conv stem step (row copies, conv0 and conv1 GEMMs on v_mfma_f32_32x32x16_bf16)",
            "achieved": tfs,
            "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s",
            "frac": tfs / MFMA_BF16_PEAK_TFS,
            "traffic": step_traffic([("k_gemm_conv", 2), ("k_gemm_reduce", 1), ("k_row_copy", 1)], "cs"),
            "traffic_note": "HBM bytes per step from the counter records: two GEMM launches, the reduce and the row copy",
            "flops_per_step": flops,
            "step_us_mean": t_step * 1e6,
            "steps_timed": len(ms),
        },
    }


def bench_cm(args):
    """The moonshine streaming encoder's attention pattern on the same
    kernels: 256 streams, 4 new frames per stream per step through six layers
    with (left, right) windows (16,4),(16,4),(16,0),(16,0),(16,4),(16,4), no
    rotation; 8 heads of 40 (the streaming-tiny model's, hidden 320; the ring
    rows are padded to 64 elements), bf16 N(0,1)*0.5."""
    import torch
    import sliding_window_cached_amd as vrt

    dev = torch.device("cuda:0")
    S, n, Hm, Dm = 256, 4, 8, 40
    groups = [(vrt.lookahead_desc(16, 4, n_layers=4, heads=Hm, head_dim=Dm), 4),
              (vrt.lookahead_desc(16, 0, n_layers=2, heads=Hm, head_dim=Dm), 2)]
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    total = args.warmup + args.steps
    pools = []
    for desc, L in groups:
        nb = vrt.state_device_bytes(desc)
        stride = (nb + 255) // 256 * 256    # each state's memory 256-byte aligned
        mem = torch.empty(S * stride, dtype=torch.uint8, device=dev)
        states = [vrt.StreamState(desc, mem[i * stride:i * stride + nb], nb, 0) for i in range(S)]
        qkv = [_randn(gen, (total, S, L, n, Hm, Dm), 0.5, dev) for _ in range(3)]
        pools.append((desc, L, mem, states, qkv, torch.empty((S, L, n, Hm, Dm), dtype=torch.bfloat16, device=dev)))

    def step(i):
        for desc, L, _, states, (Q, K, V), out in pools:
            vrt.enc_attn_feed(states, 0, L, Q[i], K[i], V[i], n, out, stream)

    device_warmup()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    every = max(1, args.timing_every or (1 if args.steps < 100 else 10))
    timed = list(range(0, args.steps, every))
    ev = dict(zip(timed, _timing_events(len(timed))))
    log(f"cm: timing {args.steps} steps of 6 lookahead layers")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        if j in ev:
            ev[j][0].record()
        step(args.warmup + j)
        if j in ev:
            ev[j][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [ev[j][0].elapsed_time(ev[j][1]) for j in timed]
    for p in pools:
        for st in p[3]:
            st.close()
    row = Hm * Dm * 2
    # per (stream, layer): q, k, v read, K/V appended, the keys of the union
    # window read (15 + F + n rows of K and V), outputs written, all at the
    # heads' 40 elements (the ring rows' padding to 64 is not counted)
    nbytes = sum(S * L * (n + 2 * n + 2 * n + 2 * (15 + max(d.lookahead - 1, 0) + n) + n) * row
                 for d, L, *_ in pools)
    t_step = sum(ms) * 1e-3 / len(ms)
    gbs = nbytes / t_step / 1e9
    return {
        "metric": "encoder frames/s through six (left, right)-window attention layers (all streams)",
        "value": S * n * args.steps / wall,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "moonshine-pattern attention: 256 streams, 4 frames per step, 6 layers with "
                        "(left, right) windows (16,4),(16,4),(16,0),(16,0),(16,4),(16,4), no RoPE, "
                        "8 heads x 40, bf16 N(0,1)*0.5; answered frames lag by 3 in the (16,4) layers",
            "streams": S, "layers": 6, "frames_per_step": n, "heads": Hm, "head_dim": Dm,
            "parallelism": "none (1 GPU)", "device_warmup_s": DEVICE_WARMUP_S,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_attn lookahead path + append + waiting-row save (two feed calls per step)",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": step_traffic([("k_attn_look", 2)], "cm"),
            "traffic_note": "HBM bytes per step from the counter records: two lookahead launches (their mean x 2)",
            "alg_bytes_per_step": nbytes,
            "step_us_mean": t_step * 1e6,
            "steps_timed": len(ms),
            "note": "windows of at most 23 keys: launch- and latency-bound, not bandwidth-bound",
        },
    }


def cpu_baseline_cm(steps: int, passes: int = 1):
    """The fp64 oracle (oracle.attention.lookahead over the frames seen so
    far, the answered rows only) for one stream through one (16,4) layer, 4
    frames per feed, the same `steps` feeds timed `passes` times (the inputs
    stay small); scaled to the six layers of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention
    from synth import qkv

    T = 16 + 4 * steps + 3
    q, k, v = qkv(7, 0, 0, T, 8, 8, 40, 0.5, "bf16")
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for _ in range(passes):
            for i in range(steps):          # a feed of 4 frames answers 4 queries, 3 frames back
                for t in range(16 + 4 * i, 16 + 4 * i + 4):
                    attention.window_rows(q[t], k[t - 15:t + 4], v[t - 15:t + 4], 1)
        el = time.perf_counter() - t0
    return {"value": 4 * steps * passes / el / 6, "unit": "frames/s", "cores": 1, "kind": "oracle",
            "sample": f"one stream, one (16,4) layer, {steps} feeds of 4 frames timed {passes} times; each answered query "
                      f"over its window (oracle.attention.window_rows, fp64 numpy, one thread), "
                      f"{el:.1f} s; divided by 6 layers"}


def cpu_baseline_conv(steps: int):
    """The fp64 oracle's streamed stem (oracle.conv.StreamStem), one stream,
    `steps` feeds of 8 mel frames, one host thread."""
    from threadpoolctl import threadpool_limits
    from oracle import conv
    from synth import conv_weights, mel_frames

    w = conv_weights(6, 128, H * D)
    mel = mel_frames(6, 0, 8 * steps, 128)
    st = conv.StreamStem(w)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for i in range(steps):
            st.feed(mel[8 * i:8 * i + 8])
        el = time.perf_counter() - t0
    return {"value": 4 * steps / el, "unit": "frames/s", "cores": 1, "kind": "oracle",
            "sample": f"one stream, {steps} feeds of 8 mel frames through oracle.conv.StreamStem "
                      f"in fp64 numpy on one thread, {el:.1f} s"}


KERNEL_DIR = os.path.join(ROOT, "sliding_window_cached_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
MFMA_BUSY_FILE = os.path.join(ROOT, "profiles", "mfma_busy.txt")
# the source file that holds each kernel a record is kept for
BLOCK_KERNELS = ("k_gemm_qkv", "k_gemm_o", "k_rmsnorm", "k_gemm_conv", "k_gemm_reduce", "k_row_copy")


def kernel_source(kernel: str) -> str:
    if kernel in BLOCK_KERNELS:
        return os.path.join(KERNEL_DIR, "vrt_block.hip")
    return os.path.join(KERNEL_DIR, "vrt_mfma.hip" if kernel == "k_attn_mfma" else "vrt_kernels.hip")


def source_sha256(path: str) -> str:
    """First 16 hex digits of the sha256 of one kernel source file: a
    recorded counter value holds only while that file is unchanged."""
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def workload_key(args, name: str) -> str:
    """Key of an encoder workload in profiles/hbm_traffic.txt: the config
    name, with an m appended for the modulo-ring variant."""
    return name + ("m" if getattr(args, "ring", "compact") == "mod" else "")


def dec_traffic():
    """Decoder step: split-K attention plus merge, per step."""
    a = measured_traffic("k_attn_dec", "c4")
    b = measured_traffic("k_dec_combine", "c4")
    return a["bytes"] + b["bytes"] if a and b else None


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the rocprofv3
    FETCH_SIZE / WRITE_SIZE runs recorded in profiles/hbm_traffic.txt
    (already scaled by the copy-kernel calibration there), or None when no
    record exists or the kernel's source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha = source_sha256(kernel_source(kernel))
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) == 5 and f[0] == kernel and f[1] == workload and f[4] == f"src_sha256={sha}":
            return {"fetch_bytes": float(f[2]), "write_bytes": float(f[3]),
                    "bytes": float(f[2]) + float(f[3])}
    return None


def step_traffic(parts, workload: str):
    """HBM bytes of one step made of several launches: sum of count x the
    per-launch record of each kernel, or None if any record is missing."""
    tot = 0.0
    for kernel, count in parts:
        r = measured_traffic(kernel, workload)
        if r is None:
            return None
        tot += count * r["bytes"]
    return tot


def measured_mfma_busy(kernel: str, workload: str):
    """Fraction of the launch the matrix cores were busy, from the rocprofv3
    SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE run recorded in
    profiles/mfma_busy.txt, or None when no record exists or the kernel's
    source changed since it was taken."""
    if not os.path.exists(MFMA_BUSY_FILE):
        return None
    sha = source_sha256(kernel_source(kernel))
    for line in open(MFMA_BUSY_FILE):
        f = line.split()
        if len(f) == 4 and f[0] == kernel and f[1] == workload and f[3] == f"src_sha256={sha}":
            return float(f[2])
    return None


def bench_copy(args):
    """Calibration: a plain device-to-device copy of 1 GiB, `steps` times
    (reads and writes exactly 2^30 bytes per launch)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"metric": "device copy bandwidth (calibration)", "value": 2 * n * args.steps / wall / 1e9,
            "unit": "GB/s", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
            "steps": args.steps}


def bench_read(args):
    """Calibration: the library's read probe streams 4 GiB (16-byte loads,
    eight in flight per thread); the practical ceiling of a read-bound
    kernel on the part, beside the nominal 8 TB/s."""
    import torch
    import sliding_window_cached_amd as vrt
    n = 1 << 32
    x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(args.warmup):
        vrt.read_probe(x, n, sink, stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        vrt.read_probe(x, n, sink, stream)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / args.steps
    return {"metric": "device streaming read bandwidth (calibration)", "value": n / t / 1e9,
            "unit": "GB/s", "frac_of_nominal": n / t / 1e9 / HBM_PEAK_GBS, "bytes_read_per_launch": n,
            "steps": args.steps, "kernel": "k_read_probe (vrt_read_probe)"}


def bench_stream(args):
    """Calibration: the vector attention kernel's tile stream with none of
    its arithmetic (vrt_tile_stream_probe).  (1) The serving step's shape:
    1024 workgroups, five heads each, 12 tiles of 8 KB K + 8 KB V per head,
    regions laid out like the rings (K and V 196608 bytes apart, heads
    393216 apart), read once per launch from HBM with that kernel's
    non-temporal loads.  (2) The same workgroups over a 753-key window as the
    kernel reads it: 13 tiles per head, the first read from row 32 and the
    last up to row 16, the other rows of those two tiles fetching the nearest
    row read (753 rows of K and V per head).  (3) The loop of (1) over 16
    regions of 64 KB that stay in L2, 200 passes, plain loads (as the GEMMs'),
    at 1, 2 and 4 workgroups per CU: the L2 -> LDS rate per CU."""
    import torch
    import sliding_window_cached_amd as vrt
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    device_warmup()

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    n_wg, heads, tiles, stride, kv_off = 1024, 5, 12, 393216, 196608
    nbytes = n_wg * heads * stride
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    t = timed(lambda: vrt.tile_stream_probe(buf, nbytes, n_wg, heads, tiles, n_wg * heads, stride, kv_off, 1,
                                            sink, stream), args.steps)
    moved = n_wg * heads * tiles * 16384
    tw = timed(lambda: vrt.tile_stream_probe(buf, nbytes, n_wg, heads, 13, n_wg * heads, stride, kv_off, 1, sink,
                                             stream, first_row=32, last_row=16), args.steps)
    rows = 32 + 11 * 64 + 17
    moved_w = n_wg * heads * rows * 256
    del buf
    small = torch.ones(16 * 65536, dtype=torch.uint8, device=dev)
    per_cu = {}
    for wpc in (1, 2, 4):
        passes = 200
        ts = timed(lambda: vrt.tile_stream_probe(small, small.numel(), 256 * wpc, 1, 4, 16, 65536, 32768, passes,
                                                 sink, stream, nontemporal=False), max(2, args.steps // 5))
        per_cu[str(wpc)] = 256 * wpc * 4 * 16384 * passes / ts / 256 / 1e9
    return {"metric": "attention tile-stream rate without arithmetic (calibration)", "value": moved / t / 1e9,
            "unit": "GB/s", "frac_of_nominal": moved / t / 1e9 / HBM_PEAK_GBS, "us_per_launch": t * 1e6,
            "bytes_per_launch": moved, "steps": args.steps,
            "serving_shape": {"workgroups": n_wg, "heads_per_workgroup": heads, "tiles_per_head": tiles,
                              "tile_bytes": 16384, "lds_stages": 2},
            "window_753_rows": {"tiles_per_head": 13, "first_row": 32, "last_row": 16, "rows_per_head": rows,
                                "us_per_launch": tw * 1e6, "bytes_of_rows_read": moved_w,
                                "gbs_of_rows_read": moved_w / tw / 1e9,
                                "note": "13 steps per head like the serving kernel's unaligned window; if the time "
                                        "follows the rows read and not the steps, this matches the 12-tile rate"},
            "l2_resident_gbs_per_cu_by_workgroups_per_cu": per_cu,
            "kernel": "k_tile_probe (vrt_tile_stream_probe)"}


def bench_gemm(args):
    """Calibration: the block's two projections at the serving shape (1024
    rows = 256 streams x 4 frames, dim 1280, bf16, no bias or residual) on
    the library's GEMM (vrt_linear, the kernel vrt_enc_block_feed runs) and
    on the vendor BLAS (torch.matmul, hipBLASLt).  Each side's `steps`
    launches are captured in one HIP graph and replayed, so the events time
    the kernels back to back, not the Python launch path."""
    import statistics
    import torch
    import sliding_window_cached_amd as vrt
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    M, K = 1024, 1280
    device_warmup()
    rows = []
    for name, N in (("q/k/v", 3 * K), ("output", K)):
        A = _randn(gen, (M, K), 1.0, dev)
        Wm = _randn(gen, (N, K), 0.03, dev)
        outs = {t: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for t in ("library", "vendor")}

        def library():
            vrt.linear(A, M, K, Wm, N, None, None, outs["library"], torch.cuda.current_stream().cuda_stream)

        def vendor():
            torch.matmul(A, Wm.t(), out=outs["vendor"])

        us = {}
        for tag, fn in (("library", library), ("vendor", vendor)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(args.steps):
                    fn()
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = []
            for _ in range(5):
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                reps.append(e0.elapsed_time(e1) * 1e3 / args.steps)
            us[tag] = statistics.median(reps)
        diff = (outs["library"].float() - outs["vendor"].float()).abs().max().item()
        flops = 2.0 * M * N * K
        rows.append({"product": name, "M": M, "N": N, "K": K,
                     "library_us": us["library"], "vendor_us": us["vendor"],
                     "library_tflops": flops / us["library"] / 1e6, "vendor_tflops": flops / us["vendor"] / 1e6,
                     "max_abs_diff_vs_vendor": diff})
    return {"metric": "projection GEMM time, library vs vendor BLAS (calibration)",
            "value": sum(r["library_us"] for r in rows), "unit": "us (q/k/v + output)",
            "higher_is_better": False, "vendor_us": sum(r["vendor_us"] for r in rows),
            "steps": args.steps, "warmup": args.warmup, "products": rows,
            "kernels": "k_gemm (vrt_linear) and the hipBLASLt kernels torch.matmul picks"}


def bench_c1(args):
    """64 streams x 32 independent layer caches, bf16 N(0,1)*0.5.  Stream i
    first ingests o_i ~ U{0..749} frames (one untimed catch-up feed) so ring
    phases and compactions are staggered, then pre-fills 750 more frames;
    each timed step feeds 4 new frames to every stream, all 32 layers, in
    one call."""
    import torch
    import sliding_window_cached_amd as vrt
    from synth import offsets

    dev = torch.device("cuda:0")
    S, L, n = 64, 32, 4
    off = [int(o) for o in offsets(1, S, 0, 750)]
    desc = enc_desc(args, L)
    nb = vrt.state_device_bytes(desc)
    mem = torch.empty(S * nb, dtype=torch.uint8, device=dev)
    states = [vrt.StreamState(desc, mem[i * nb:(i + 1) * nb], nb, 0) for i in range(S)]
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    log("c1: staggered catch-up feeds and a 750-frame pre-fill per stream")
    blk = [_randn(gen, (1, L, 750, H, D), 0.5, dev) for _ in range(3)]
    ob = torch.empty_like(blk[0])
    for i in range(S):
        for m in ([off[i]] if off[i] else []) + [750]:
            vrt.enc_attn_feed([states[i]], 0, L, *(x[:, :, :m].contiguous() for x in blk), m, ob, stream)
    torch.cuda.synchronize()
    del blk, ob
    total = args.warmup + args.steps
    log(f"c1: drawing inputs for {total} steps into HBM")
    Q, K, V = (_randn(gen, (total, S, L, n, H, D), 0.5, dev) for _ in range(3))
    out = torch.empty((S, L, n, H, D), dtype=torch.bfloat16, device=dev)
    device_warmup()
    for i in range(args.warmup):
        vrt.enc_attn_feed(states, 0, L, Q[i], K[i], V[i], n, out, stream)
    torch.cuda.synchronize()
    plan = []
    nkv = [st.query(0)[1] for st in states]
    for j in range(args.steps):
        step = []
        for i in range(S):
            _, after, nc = vrt.ring_advance(desc, 0, nkv[i], n)
            step.append((after - n, nc))
            nkv[i] = after
        plan.append(step)
    ev = _timing_events(args.steps)
    log(f"c1: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        i = args.warmup + j
        vrt.set_attn_events(ev[j][0], ev[j][1])
        vrt.enc_attn_feed(states, 0, L, Q[i], K[i], V[i], n, out, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    vrt.set_attn_events()
    attn_ms = [a.elapsed_time(b) for a, b in ev]

    # the same kind of step as 32 per-layer calls of 64 streams each (the
    # order in which a real encoder runs its layers: one layer's output is the
    # next one's input), on the wall clock, continuing the same streams
    nl_steps = min(args.steps, max(0, args.per_layer_steps))
    Qp, Kp, Vp = (x[args.warmup:args.warmup + nl_steps].transpose(1, 2).contiguous() for x in (Q, K, V))
    out_l = torch.empty((S, 1, n, H, D), dtype=torch.bfloat16, device=dev)
    log(f"c1: timing {nl_steps} steps as {L} per-layer calls each")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for j in range(nl_steps):
        for l in range(L):
            vrt.enc_attn_feed(states, l, 1, Qp[j, l], Kp[j, l], Vp[j, l], n, out_l, stream)
    torch.cuda.synchronize()
    wall_l = max(time.perf_counter() - t1, 1e-9)
    del Qp, Kp, Vp
    for st in states:
        st.close()
    nbytes = [L * sum(attn_work(k, n)[0] for k, _ in step) for step in plan]
    t_attn = sum(attn_ms) * 1e-3
    gbs = sum(nbytes) / t_attn / 1e9
    return {
        "metric": METRIC,
        "value": S * n * args.steps / wall,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"64 streams x 32 layers, 20 heads x 64, window 750, {ring_words(desc)}, bf16 N(0,1)*0.5, "
                        "staggered ring phases (catch-up of U{0..749} frames, then 750), 4 frames per "
                        "stream per step, all layers in one call",
            "streams": S, "layers": L, "frames_per_step": n, "ring_slots": desc.ring_slots,
            "ring": args.ring, "parallelism": "none (1 GPU)", "device_warmup_s": DEVICE_WARMUP_S,
            "compactions_timed": sum(nc for step in plan for _, nc in step),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_attn (vector path: fused RoPE + append + attention, 2048 units per launch)",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": (measured_traffic("k_attn", workload_key(args, "c1")) or {}).get("bytes"),
            "alg_bytes_per_launch": nbytes[-1],
            "launch_us_mean": t_attn / len(attn_ms) * 1e6,
            "launches_timed": len(attn_ms),
        },
        "step_hbm_frac": sum(nbytes) / wall / 1e9 / HBM_PEAK_GBS,
        "per_layer_calls": None if nl_steps == 0 else {
            "steps": nl_steps, "ms_per_step": wall_l * 1e3 / nl_steps,
            "value": S * n * nl_steps / wall_l,
            "note": "each step as 32 calls (one layer of all 64 streams each, 64 units per launch), "
                    "wall clock",
        },
    }


def mfma_band(avail: int, p0: int, n: int, qtile: int = 128, qw: int = 32):
    """(visible, computed) (query, key) pairs of one unit's matrix-core
    attention: visible = the keys in each query's window; computed = the
    32-key x 32-query blocks the kernel runs, a wave skipping the half-tiles
    of the absolute 64-key grid that hold no key of any of its queries."""
    visible = sum(q - max(avail, q - W + 1) + 1 for q in range(p0, p0 + n))
    computed = 0
    for qc in range((n + qtile - 1) // qtile):
        pq0 = p0 + qc * qtile
        nq = min(qtile, n - qc * qtile)
        wlo, whi = max(avail, pq0 - W + 1), pq0 + nq - 1
        t0 = (wlo // 64) * 64
        for w0 in range(0, nq, qw):
            first, last = pq0 + w0, pq0 + min(nq, w0 + qw) - 1
            blo, bhi = max(avail, first - W + 1) - t0, last - t0
            kb = 0
            while kb <= whi - t0:
                if kb + 31 >= blo and kb <= bhi:
                    computed += 32 * qw
                kb += 32
    return visible, computed


def c3_schedule(T=15300, B=512):
    return [min(B, T - t) for t in range(0, T, B)]


def bench_c3(args):
    import torch
    import sliding_window_cached_amd as vrt

    dev = torch.device("cuda:0")
    L, start = 32, 0
    sched = c3_schedule()
    desc = enc_desc(args, L)
    nb = vrt.state_device_bytes(desc)
    mem = torch.empty(nb, dtype=torch.uint8, device=dev)
    st = vrt.StreamState(desc, mem, nb, start)
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    log(f"c3: drawing 32 layers x {sum(sched)} frames into HBM ({len(sched)} batches)")
    batches = [tuple(_randn(gen, (1, L, m, H, D), 1.0, dev) for _ in range(3)) for m in sched]
    outs = {m: torch.empty((1, L, m, H, D), dtype=torch.bfloat16, device=dev) for m in set(sched)}

    def feed(b):
        q, k, v = batches[b]
        vrt.enc_attn_feed([st], 0, L, q, k, v, sched[b], outs[sched[b]], stream)

    # warmup: whole sequences from a reset ring
    device_warmup()
    b = 0
    for _ in range(args.warmup):
        feed(b)
        b += 1
        if b == len(sched):
            b = 0
            st.reset(start)
    torch.cuda.synchronize()

    # host mirror of the ring each timed batch's attention sees
    plan = []
    bb, base, nkv = b, *st.query(0)
    for j in range(args.steps):
        m = sched[bb]
        base, nkv_after, _ = vrt.ring_advance(desc, base, nkv, m)
        plan.append((bb, m, nkv_after - m, base))
        nkv = nkv_after
        bb += 1
        if bb == len(sched):
            bb, base, nkv = 0, start, 0

    ev = _timing_events(args.steps)
    log(f"c3: timing {args.steps} batches")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j, (bj, m, _, _) in enumerate(plan):
        vrt.set_attn_events(ev[j][0], ev[j][1])
        feed(bj)
        if bj == len(sched) - 1:
            st.reset(start)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    vrt.set_attn_events()
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    st.close()

    frames = sum(m for _, m, _, _ in plan)
    work = [attn_work(k, m) for _, m, k, _ in plan]
    band = [mfma_band(base, base + k, m) for _, m, k, base in plan]
    nbytes = sum(L * attn_kernel_bytes(k, m) for _, m, k, _ in plan)
    flops = sum(L * w[1] for w in work)
    t_attn = sum(attn_ms) * 1e-3
    tflops = flops / t_attn / 1e12
    gbs = nbytes / t_attn / 1e9
    full = [(a, L * attn_work(k, m)[1]) for a, (_, m, k, _) in zip(attn_ms, plan) if m == 512 and k >= W]
    return {
        "metric": METRIC,
        "value": frames / wall,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"catch-up: 1 stream x 32 layers, 20 heads x 64, window 750, {ring_words(desc)}, "
                        "15300 frames as 29 x 512 + 452 (max batch 512), bf16 N(0,1); one step = "
                        "one batch through all 32 layers",
            "streams": 1, "layers": L, "frames": sum(sched), "max_batch": 512, "heads": H,
            "head_dim": D, "window": W, "ring_slots": desc.ring_slots, "ring": args.ring,
            "parallelism": "none (1 GPU)", "device_warmup_s": DEVICE_WARMUP_S,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_attn_mfma (matrix path: S^T = K Q^T and O^T += V^T P^T on "
                      "v_mfma_f32_32x32x16_bf16)",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": (measured_traffic("k_attn_mfma", workload_key(args, "c3")) or {}).get("bytes"),
            "bytes_model": "fused minimum per unit-batch (n q rows + 2 (old + n) K/V rows + n out rows) "
                           "* H * d * 2 B, old = min(n_kv, 749)",
            "alg_flops_per_launch_full_window": full[0][1] if full else None,
            "launch_us_mean": t_attn / len(attn_ms) * 1e6,
            "launch_us_mean_full_window": (sum(a for a, _ in full) / len(full) * 1e3) if full else None,
            "launches_timed": len(attn_ms),
            "mfma_achieved_tflops": tflops,
            "mfma_frac": tflops / MFMA_BF16_PEAK_TFS,
            "mfma_busy_counter": measured_mfma_busy("k_attn_mfma", workload_key(args, "c3")),
            "band_efficiency": sum(v for v, _ in band) / sum(c for _, c in band),
            "note": "the binding roof is HBM: the fused minimum bytes take longer at 8 TB/s than the "
                    "algorithmic flops (4*d*H per (query, visible key)) at 2.5 PFLOP/s, about 216 flop/B "
                    "against the 312 flop/B bf16 ridge; mfma_frac is the flop rate against the bf16 peak "
                    "and mfma_busy_counter = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 "
                    "SIMDs) from the rocprofv3 counter run of the same workload; band_efficiency = "
                    "visible (query, key) pairs / pairs in the 32 x 32 score blocks the kernel computes",
        },
    }


def bench_c4(args):
    """Decoder step: 32 streams x 26 layers, GQA 32 query / 8 kv heads, head_dim
    128, window 8192, modulo ring, bf16 N(0,1).  Contexts: 24 streams
    uniform in [39, 8192], 8 streams uniform in [8193, 10269] (past the ring
    wrap).  Each cache is filled through the library (untimed): a 39-token
    prefill, prefills of up to 512 tokens up to the wrap, then single-token
    steps; the filled keys are random (one 512-token block of inputs reused).
    One step = one token for every stream through all 26 layers (split-K
    attention over the window, then the merge)."""
    import torch
    import sliding_window_cached_amd as vrt
    from synth import offsets

    dev = torch.device("cuda:0")
    S, L, HQ, HK, DD, WIN = 32, 26, 32, 8, 128, 8192
    ctx = [int(c) for c in offsets(4, 24, 39, 8193)] + [int(c) for c in offsets(4, 8, 8193, 10270)]
    desc = vrt.dec_desc(dtype=vrt.BF16, n_layers=L)
    nb = vrt.state_device_bytes(desc)
    mem = torch.empty(S * nb, dtype=torch.uint8, device=dev)
    states = [vrt.StreamState(desc, mem[i * nb:(i + 1) * nb], nb, 0) for i in range(S)]
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    B = 512
    qb = _randn(gen, (1, L, B, HQ, DD), 1.0, dev)
    kb = _randn(gen, (1, L, B, HK, DD), 1.0, dev)
    vb = _randn(gen, (1, L, B, HK, DD), 1.0, dev)
    ob = torch.empty_like(qb)
    ws1 = vrt.dec_workspace_bytes(desc, 1, L, 1)
    wsb = vrt.dec_workspace_bytes(desc, S, L, 1)
    ws = torch.empty(max(ws1, wsb) // 4 + 1, dtype=torch.float32, device=dev)
    log(f"c4: filling 32 decoder caches (26 layers) to contexts {min(ctx)}..{max(ctx)}")
    t_fill = time.perf_counter()
    for i in range(S):
        n = 0
        for m in [39] + [B] * 64:
            m = min(m, min(ctx[i], WIN) - n)
            if m <= 0:
                break
            def sl(x, m=m):
                return x[:, :, :m].contiguous()
            vrt.dec_attn_step([states[i]], 0, L, sl(qb), sl(kb), sl(vb), m, ob, stream=stream)
            n += m
    # single-token steps past the wrap, all long streams together
    q1, k1, v1, o1 = (x[:, :, :1].expand(S, L, 1, x.shape[3], DD).contiguous()
                      for x in (qb, kb, vb, ob))
    while True:
        need = [i for i in range(S) if states[i].query(0)[1] < ctx[i]]
        if not need:
            break
        k = len(need)
        vrt.dec_attn_step([states[i] for i in need], 0, L, q1[:k], k1[:k], v1[:k], 1, o1[:k], ws,
                          wsb, stream)
    torch.cuda.synchronize()
    log(f"c4: filled in {time.perf_counter() - t_fill:.1f} s")
    total = args.warmup + args.steps
    Q = _randn(gen, (total, S, L, 1, HQ, DD), 1.0, dev)
    K = _randn(gen, (total, S, L, 1, HK, DD), 1.0, dev)
    V = _randn(gen, (total, S, L, 1, HK, DD), 1.0, dev)
    out = torch.empty((S, L, 1, HQ, DD), dtype=torch.bfloat16, device=dev)
    device_warmup()
    for j in range(args.warmup):
        vrt.dec_attn_step(states, 0, L, Q[j], K[j], V[j], 1, out, ws, wsb, stream)
    torch.cuda.synchronize()
    seen = []   # keys each unit's step attends to
    for j in range(args.steps):
        seen.append([min(WIN, states[i].query(0)[1] + j + 1) for i in range(S)])
    ev = _timing_events(args.steps)
    log(f"c4: timing {args.steps} decode steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        i = args.warmup + j
        vrt.set_attn_events(ev[j][0], ev[j][1])
        vrt.dec_attn_step(states, 0, L, Q[i], K[i], V[i], 1, out, ws, wsb, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    vrt.set_attn_events()
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    for st in states:
        st.close()
    # algorithmic bytes of one step: every unit reads the K and V rows of its
    # window (8 kv heads x 128 x bf16) and its q; writes its new K/V row and out
    row = HK * DD * 2
    nbytes = [L * sum(2 * n * row + (2 * HQ * DD * 2) + 2 * row for n in w) for w in seen]
    t_attn = sum(attn_ms) * 1e-3
    gbs = sum(nbytes) / t_attn / 1e9
    return {
        "metric": "decoder tokens/s through the cached window-8192 GQA step (all streams, 26 layers each)",
        "value": S * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decoder step: 32 streams x 26 layers, GQA 32/8 heads x 128, window 8192, "
                        "modulo ring 8192, bf16 N(0,1); contexts 24 x U[39, 8192] and 8 x "
                        "U[8193, 10269]; one step = one token per stream",
            "streams": S, "layers": L, "heads_q": HQ, "heads_kv": HK, "head_dim": DD, "window": WIN,
            "contexts": ctx, "parallelism": "none (1 GPU)", "device_warmup_s": DEVICE_WARMUP_S,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_attn split-K (kv heads x 2048-key splits) + k_dec_combine",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": dec_traffic(),
            "alg_bytes_per_launch": nbytes[-1],
            "launch_us_mean": t_attn / len(attn_ms) * 1e6,
            "launches_timed": len(attn_ms),
        },
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="default: c2 1000, c3 300")
    ap.add_argument("--warmup", type=int, default=None, help="default: c2 20, c3 30")
    ap.add_argument("--config", default="c2",
                    choices=["c1", "c2", "c2b", "c3", "c4", "cs", "cm", "copy", "read", "gemm", "stream"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--device-warmup", type=float, default=DEVICE_WARMUP_S,
                    help="seconds of untimed HBM streaming and bf16 products before the warmup steps "
                         "(0: none; profiler runs use 0 to keep the trace small)")
    ap.add_argument("--per-layer-steps", type=int, default=50,
                    help="c1: also time this many steps as 32 per-layer calls (0: skip; "
                         "profiler runs skip them)")
    ap.add_argument("--ring", default="compact", choices=["compact", "mod"],
                    help="encoder configs: compacting ring (the pages') or modulo ring")
    ap.add_argument("--timing-every", type=int, default=None,
                    help="c2: record the attention-kernel events on every N-th timed step "
                         "(default: every step below 100 steps, else every 10th)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (--gpus 1): streams are independent and would "
              "shard across GPUs with no exchange; a single GPU is run and reported.",
              file=sys.stderr)
        sys.exit(2)
    globals()["DEVICE_WARMUP_S"] = max(0.0, args.device_warmup)
    if not args.no_cpu_baseline and args.config in ("c1", "c2", "c3"):
        start_cpu_pool()    # before anything touches the GPU
    if args.config == "copy":
        args.steps = 20 if args.steps is None else args.steps
        args.warmup = 2 if args.warmup is None else args.warmup
        print(json.dumps(bench_copy(args)), flush=True)
        return
    if args.config == "read":
        args.steps = 20 if args.steps is None else args.steps
        args.warmup = 2 if args.warmup is None else args.warmup
        print(json.dumps(bench_read(args)), flush=True)
        return
    if args.config == "stream":
        args.steps = 20 if args.steps is None else args.steps
        args.warmup = 2 if args.warmup is None else args.warmup
        print(json.dumps(bench_stream(args)), flush=True)
        return
    if args.config == "gemm":
        args.steps = 50 if args.steps is None else args.steps
        args.warmup = 5 if args.warmup is None else args.warmup
        print(json.dumps(bench_gemm(args)), flush=True)
        return
    if args.config == "c2":
        args.steps = 1000 if args.steps is None else args.steps
        args.warmup = 20 if args.warmup is None else args.warmup
        res = bench_c2(args)
    elif args.config == "c2b":
        args.steps = 300 if args.steps is None else args.steps
        args.warmup = 10 if args.warmup is None else args.warmup
        res = bench_c2b(args)
    elif args.config == "cs":
        args.steps = 300 if args.steps is None else args.steps
        args.warmup = 10 if args.warmup is None else args.warmup
        res = bench_cs(args)
    elif args.config == "cm":
        args.steps = 300 if args.steps is None else args.steps
        args.warmup = 10 if args.warmup is None else args.warmup
        res = bench_cm(args)
    elif args.config == "c1":
        args.steps = 200 if args.steps is None else args.steps
        args.warmup = 10 if args.warmup is None else args.warmup
        res = bench_c1(args)
    elif args.config == "c3":
        args.steps = 300 if args.steps is None else args.steps
        args.warmup = 30 if args.warmup is None else args.warmup
        res = bench_c3(args)
    else:
        args.steps = 100 if args.steps is None else args.steps
        args.warmup = 5 if args.warmup is None else args.warmup
        res = bench_c4(args)
    if args.no_cpu_baseline:
        res["cpu_baseline"] = None
    else:
        log("cpu baseline: timing the fp64 oracle on a bounded sample")
        from synth import offsets
        if args.config == "c2":
            res["cpu_baseline"] = cpu_baseline(1, W, 1000, 4, 0.5, offsets(2, 16, 10 ** 4, 10 ** 6),
                                               "steady-state sample", seed=2)
        elif args.config == "c2b":
            res["cpu_baseline"] = cpu_baseline_block(750)
        elif args.config == "cs":
            res["cpu_baseline"] = cpu_baseline_conv(450)
        elif args.config == "cm":
            res["cpu_baseline"] = cpu_baseline_cm(10000, passes=8)
        elif args.config == "c1":
            res["cpu_baseline"] = cpu_baseline(32, W, 1000, 4, 0.5, [0], "staggered-streams sample", seed=1)
        elif args.config == "c3":
            res["cpu_baseline"] = cpu_baseline(32, 0, 10, 512, 1.0, [0], "catch-up sample", seed=3)
        else:
            res["cpu_baseline"] = cpu_baseline_dec(res["config"]["contexts"])
    if CPU_POOL is not None:
        CPU_POOL[0].terminate()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
