"""GPU hazard test: no kernel reads memory outside what it has written.

Every byte of state memory (rings, waiting query rows), of the decoder's
split workspace and of the offline scratch is filled with 0xFF before the
first call (a NaN in bf16 and in fp32), and the run is repeated over memory
filled with zeros.  A read of any slot outside a query's window, of a ring
row not yet written, of a stale row after a compaction or of a split partial
that was never written would carry the NaN into an output (a weight of zero
times NaN is still NaN), so the bar is: outputs finite and bit-identical to
the zero-filled run, on both attention paths, in bf16 and fp32, across
compactions, on every cache kind (streaming-plan page, "Per-hook behavior":
reset clears the streaming state but keeps the allocations, so a state's
memory holds whatever an earlier stream left there)."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from synth import qkv

from gpu_util import DEV, Pool, empty, host, run_feeds, say, seqs, stream, to_dev

pytestmark = pytest.mark.gpu


def _filled_pool(desc, S, starts, byte):
    pool = Pool(desc, S, starts)
    pool.mem.fill_(byte)
    return pool


def _both(run):
    outs = []
    for byte in (0xFF, 0x00):
        outs.append(run(byte))
    a, b = outs
    assert np.isfinite(a).all(), "a NaN from unwritten memory reached an output"
    assert np.array_equal(a, b)
    return a


@pytest.mark.parametrize("kind,dtype,sizes,T", [
    (vrt.ENC_RING, vrt.BF16, [4], 1800),          # vector path, fused append, one compaction
    (vrt.ENC_RING, vrt.BF16, [100], 2600),        # matrix path, separate append, compactions
    (vrt.ENC_RING, vrt.F32, [5], 1700),           # fp32 vector path
    (vrt.ENC_RING, vrt.BF16, [3, 64, 1, 200], 1900),   # both paths in one stream
    (vrt.ENC_MODRING, vrt.BF16, [4], 1800),
    (vrt.ENC_MODRING, vrt.BF16, [100], 2600),
])
def test_encoder_reads_only_written_rows(kind, dtype, sizes, T):
    S, L, H, d = 2, 2, 20, 64
    desc = vrt.enc_desc(dtype=dtype, n_layers=L, kind=kind)
    starts = [3, 777_777]
    q, k, v = seqs(90, S, L, T, H, d, 0.5, dtype)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))

    def run(byte):
        pool = _filled_pool(desc, S, starts, byte)
        say(f"kind {kind} dtype {dtype} feeds {sizes}: state memory filled with {byte:#04x}")
        out = host(run_feeds(pool, range(S), 0, L, qd, kd, vd, sizes))
        pool.close()
        return out

    _both(run)


def test_decoder_reads_only_written_slots_and_partials():
    T, L = 700, 2
    desc = vrt.dec_desc(window=256, ring_slots=256, n_layers=L)
    qs, ks, vs = zip(*(qkv(91, 0, l, T, 32, 8, 128, 1.0, "bf16") for l in range(L)))
    qd, kd, vd = (to_dev(np.stack(x)[None], vrt.BF16) for x in (qs, ks, vs))
    sched = [39, 20] + [1] * (T - 59)
    wsb = vrt.dec_workspace_bytes(desc, 1, L, 1)

    def run(byte):
        pool = _filled_pool(desc, 1, [0], byte)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        ws.fill_(byte)
        say(f"decoder window 256: state and workspace filled with {byte:#04x}")
        out = torch.empty_like(qd)
        t = 0
        for n in sched:
            o = torch.empty_like(qd[:, :, t:t + n])
            vrt.dec_attn_step(pool.states, 0, L, qd[:, :, t:t + n].contiguous(),
                              kd[:, :, t:t + n].contiguous(), vd[:, :, t:t + n].contiguous(), n, o,
                              ws, wsb, stream())
            out[:, :, t:t + n] = o
            t += n
        torch.cuda.synchronize()
        pool.close()
        return host(out)

    _both(run)


@pytest.mark.parametrize("dtype,T", [(vrt.BF16, 900), (vrt.BF16, 20), (vrt.F32, 900)])
def test_offline_reads_only_written_scratch(dtype, T):
    H, d = 20, 64
    desc = vrt.enc_desc(dtype=dtype)
    q, k, v = seqs(92, 1, 1, T, H, d, 0.5, dtype)
    qd, kd, vd = (to_dev(x[0, 0], dtype) for x in (q, k, v))
    sb = vrt.offline_scratch_bytes(desc, T)

    def run(byte):
        scratch = torch.empty(sb, dtype=torch.uint8, device=DEV)
        scratch.fill_(byte)
        out = empty((T, H, d), dtype)
        say(f"offline T={T} dtype {dtype}: scratch filled with {byte:#04x}")
        vrt.enc_attn_offline(desc, qd, kd, vd, T, 5000, out, scratch, sb, stream())
        torch.cuda.synchronize()
        return host(out)

    _both(run)


@pytest.mark.parametrize("d", [40, 64])
def test_lookahead_reads_only_written_rows(d):
    S, L, T, H = 2, 1, 600, 8
    desc = vrt.lookahead_desc(16, 4, n_layers=L, head_dim=d)
    q, k, v = seqs(93, S, L, T, H, d, 1.0, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))

    def run(byte):
        pool = _filled_pool(desc, S, [0, 0], byte)
        say(f"lookahead (16, 4), head_dim {d}: state memory filled with {byte:#04x}")
        outs, t = [], 0
        for m in [1, 4, 7, 64, 3] * 100:
            if t >= T:
                break
            m = min(m, T - t)
            _, nkv = pool.states[0].query(0)
            n_out = vrt.attn_out_frames(desc, nkv, m)
            qc, kc, vc = (x[:, :, t:t + m].contiguous() for x in (qd, kd, vd))
            oc = torch.empty_like(qc)
            vrt.enc_attn_feed(pool.states, 0, L, qc, kc, vc, m, oc, stream())
            if n_out:
                outs.append(oc[:, :, :n_out].clone())
            t += m
        torch.cuda.synchronize()
        pool.close()
        return host(torch.cat(outs, dim=2))

    _both(run)
