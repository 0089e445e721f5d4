"""Parity at the full benchmark sizes, in the launch configuration bench.py
times, on sampled outputs the oracle computes one by one.

Steady-state serving (vector path): 256 streams x 1 layer, bf16 N(0,1)*0.5,
start positions U[1e4, 1e6), rings pre-filled with 750 frames, then 4-frame
feeds of all 256 streams in one call, across a compaction.
Catch-up (matrix path): 1 stream x 32 layers, bf16 N(0,1), 15300 frames in
29 feeds of 512 and one of 452, compactions between feeds; three layers are
also run offline over the whole 15300 frames and must match bit for bit.

Inputs are drawn on the GPU from seeded generators; the rows checked and the
windows they read are copied to the host for the oracle.  Bar: max-abs error
<= 2e-2 (bf16), plus ring metadata equal to the oracle's ring model."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention
from oracle.ring import EncRing
from synth import offsets

from gpu_util import DEV, check_close, say, stream

pytestmark = pytest.mark.gpu
THETA = 1.0e6
H, D, W = 20, 64, 750


def randn(gen, shape, scale):
    x = torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32)
    return (x * scale).to(torch.bfloat16)


def as_np(t):
    return t.float().cpu().numpy()


def test_steady_state_256_streams_sampled():
    S, n, steps = 256, 4, 220
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=1)
    starts = offsets(2, S, 10 ** 4, 10 ** 6)
    nb = vrt.state_device_bytes(desc)
    mem = torch.empty(S * nb, dtype=torch.uint8, device=DEV)
    states = [vrt.StreamState(desc, mem[i * nb:(i + 1) * nb], nb, int(starts[i])) for i in range(S)]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(20)
    T = W + steps * n
    say(f"steady state: 256 streams, pre-fill 750, {steps} feeds of 4")
    q, k, v = (randn(gen, (S, 1, T, H, D), 0.5) for _ in range(3))
    out = torch.empty_like(q)
    o = torch.empty((S, 1, W, H, D), dtype=torch.bfloat16, device=DEV)
    vrt.enc_attn_feed(states, 0, 1, q[:, :, :W].contiguous(), k[:, :, :W].contiguous(),
                      v[:, :, :W].contiguous(), W, o, stream())
    out[:, :, :W] = o
    for i in range(steps):
        a = W + i * n
        qc, kc, vc = (x[:, :, a:a + n].contiguous() for x in (q, k, v))
        oc = torch.empty_like(qc)
        vrt.enc_attn_feed(states, 0, 1, qc, kc, vc, n, oc, stream())
        out[:, :, a:a + n] = oc
    torch.cuda.synchronize()
    r = EncRing()
    for s in (0, 77, 255):
        r.reset(int(starts[s]))
        r.feed(W)
        for i in range(steps):
            r.feed(n)
        assert states[s].query(0) == (r.abs_base, r.n_kv), s
    assert len(r.events) == 1   # one compaction inside the run (before frame 1534)
    rng = np.random.default_rng(5)
    for s in [0, 1, 128, 255] + list(rng.choice(S, 4, replace=False)):
        ts = sorted({W - 1, W, 1533, 1534, 1535, 1537, T - 1} | set(rng.integers(W, T, 6).tolist()))
        qs, ks, vs = (as_np(x[s, 0]) for x in (q, k, v))
        ref = attention.windowed_at(qs, ks, vs, int(starts[s]), W, THETA, ts)
        check_close(as_np(out[s, 0])[ts], ref, vrt.BF16, f"stream {s} sampled")
    for st in states:
        st.close()


def test_catchup_32_layers_sampled():
    L, start = 32, 0
    sched = [min(512, 15300 - t) for t in range(0, 15300, 512)]
    T = sum(sched)
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=L)
    nb = vrt.state_device_bytes(desc)
    mem = torch.empty(nb, dtype=torch.uint8, device=DEV)
    st = vrt.StreamState(desc, mem, nb, start)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(30)
    say(f"catch-up: 32 layers x {T} frames in {len(sched)} feeds")
    q, k, v = (randn(gen, (1, L, T, H, D), 1.0) for _ in range(3))
    out = torch.empty_like(q)
    t = 0
    for m in sched:
        qc, kc, vc = (x[:, :, t:t + m].contiguous() for x in (q, k, v))
        oc = torch.empty_like(qc)
        vrt.enc_attn_feed([st], 0, L, qc, kc, vc, m, oc, stream())
        out[:, :, t:t + m] = oc
        t += m
    torch.cuda.synchronize()
    r = EncRing()
    r.reset(start)
    for m in sched:
        r.feed(m)
    assert len(r.events) == 27
    for l in range(L):
        assert st.query(l) == (r.abs_base, r.n_kv), l
    # the whole sequence offline (T = 15300, the same matrix-path kernel over a
    # linear scratch): bit-identical to the 512-frame feeds with their 27
    # compactions, on three layers (streaming-plan page, Verification item 1)
    sb = vrt.offline_scratch_bytes(desc, T)
    scratch = torch.empty(sb, dtype=torch.uint8, device=DEV)
    off = torch.empty((T, H, D), dtype=torch.bfloat16, device=DEV)
    for l in (0, 13, 31):
        say(f"offline T={T}, layer {l}")
        vrt.enc_attn_offline(desc, q[0, l], k[0, l], v[0, l], T, start, off, scratch, sb, stream())
        torch.cuda.synchronize()
        assert torch.equal(off, out[0, l]), f"offline != streamed, layer {l}"
    del scratch, off
    rng = np.random.default_rng(6)
    for l in (0, 13, 31):
        ts = sorted({0, 511, 512, 1535, 1536, 7000, T - 453, T - 452, T - 1}
                    | set(rng.integers(0, T, 8).tolist()))
        lo = max(0, min(ts) - W)
        qs, ks, vs = (as_np(x[0, l, lo:]) for x in (q, k, v))
        ref = attention.windowed_at(qs, ks, vs, start + lo, W, THETA, [t - lo for t in ts])
        check_close(as_np(out[0, l])[ts], ref, vrt.BF16, f"layer {l} sampled")
    st.close()
