"""GPU parity at the widest query rows the vector attention kernel holds:
fp32 at head_dim 128, where a workgroup's 16 query rows of one head take
8 KB of LDS (16 x 512 bytes), more than any other storage type and width.
Both the rotated queries and the staged output rows live there.

Encoder: feeds of 16 or more frames (16 rows per head) through a compacting
ring, bit-identical to one offline pass and within the fp32 tolerance of the
fp64 oracle.  Decoder: GQA 8/2 (group 4), a 39-token prefill (4 tokens x 4
q heads = 16 rows per kv head) and single-token steps, a 256-slot ring
bit-identical to a 1024-slot buffer that never wraps, both against the
oracle."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention
from synth import qkv

from gpu_util import DEV, Pool, check_close, empty, host, run_feeds, say, stream, to_dev

pytestmark = pytest.mark.gpu
THETA = 1.0e6


def test_encoder_fp32_head_dim_128_wide_rows():
    H, d, W, T, start = 4, 128, 200, 700, 3000
    desc = vrt.enc_desc(dtype=vrt.F32, n_layers=1, heads=H, head_dim=d, window=W, ring_slots=W + 96,
                        max_batch=64)
    q, k, v = qkv(41, 0, 0, T, H, H, d, 1.0, "f32")
    qd, kd, vd = (to_dev(x[None, None], vrt.F32) for x in (q, k, v))
    sizes = [16, 20, 3, 33, 64, 17, 1, 16] * 4
    sizes += [T - sum(sizes)]
    assert sizes[-1] > 0
    say(f"fp32 hd128 encoder: {len(sizes)} feeds, window {W}, ring {W + 96}")
    pool = Pool(desc, 1, [start])
    out = host(run_feeds(pool, [0], 0, 1, qd, kd, vd, sizes))[0, 0]
    assert pool.states[0].query(0)[0] + pool.states[0].query(0)[1] == start + T
    pool.close()
    sb = vrt.offline_scratch_bytes(desc, T)
    scratch = torch.empty(sb, dtype=torch.uint8, device=DEV)
    off = empty((T, H, d), vrt.F32)
    vrt.enc_attn_offline(desc, qd[0, 0], kd[0, 0], vd[0, 0], T, start, off, scratch, sb, stream())
    torch.cuda.synchronize()
    assert np.array_equal(host(off), out), "chunked feeds differ from the offline pass"
    ref = attention.windowed(q, k, v, start, W, THETA)
    check_close(out, ref, vrt.F32, "fp32 hd128 encoder vs oracle")


def _dec_run(desc, q, k, v, schedule):
    T = q.shape[0]
    pool = Pool(desc, 1, [0])
    qd, kd, vd = (to_dev(x, desc.dtype) for x in (q, k, v))
    ws_b = vrt.dec_workspace_bytes(desc, 1, 1, 1)
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


def test_decoder_fp32_head_dim_128_prefill_wide_rows():
    T, W = 420, 256
    q, k, v = qkv(42, 0, 0, T, 8, 2, 128, 1.0, "f32")
    sched = [39, 20] + [1] * (T - 59)
    mk = lambda slots: vrt.dec_desc(dtype=vrt.F32, heads_q=8, heads_kv=2, head_dim=128, window=W,
                                     ring_slots=slots)
    say("fp32 hd128 decoder, GQA 8/2: ring 256")
    ring = _dec_run(mk(256), q, k, v, sched)
    say("fp32 hd128 decoder, GQA 8/2: linear 1024")
    lin = _dec_run(mk(1024), q, k, v, sched)
    assert np.array_equal(ring, lin), "ring and never-wrapping buffer differ"
    ref = attention.windowed(q, k, v, 0, W, THETA)
    check_close(ring, ref, vrt.F32, "fp32 hd128 decoder vs oracle")
