"""GPU parity of (left, right) lookahead windows without rotation (the
moonshine streaming encoder's per-layer masks), through the C ABI, against
the fp64 oracle (oracle.attention.lookahead).

A query is answered once the frames it sees past itself have been fed; the
queries still waiting keep their q rows in the state.  Bars: outputs for
every answered query are bit-identical under any chunking (1, 4, 7, 64 and
512 frames) and equal to the offline pass; within the gpu_util tolerances
of the oracle; states holding different numbers of waiting queries are
refused in one call."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention

from gpu_util import DEV, Pool, check_close, host, say, seqs, stream, to_dev

pytestmark = pytest.mark.gpu


def _feed_all(pool, idx, L, qd, kd, vd, sizes):
    """Feed [S][L][T][H][d] in chunks; return the answered outputs, in order."""
    T = qd.shape[2]
    states = [pool.states[i] for i in idx]
    outs, t, i = [], 0, 0
    while t < T:
        m = min(sizes[i % len(sizes)], T - t)
        _, nkv = states[0].query(0)
        n_out = vrt.attn_out_frames(pool.desc, nkv, m)
        qc, kc, vc = (x[:, :, t:t + m].contiguous() for x in (qd, kd, vd))
        oc = torch.empty_like(qc)
        vrt.enc_attn_feed(states, 0, L, qc, kc, vc, m, oc, stream())
        if n_out:
            outs.append(oc[:, :, :n_out].clone())
        t, i = t + m, i + 1
    torch.cuda.synchronize()
    return host(torch.cat(outs, dim=2))


@pytest.mark.parametrize("dtype,left,right,d", [
    (vrt.BF16, 16, 4, 40), (vrt.F32, 16, 4, 40), (vrt.BF16, 16, 0, 40), (vrt.BF16, 16, 1, 40),
    (vrt.BF16, 100, 9, 40), (vrt.BF16, 16, 4, 64), (vrt.F32, 100, 9, 64), (vrt.BF16, 16, 4, 8)])
def test_lookahead_chunkings_offline_and_oracle(dtype, left, right, d):
    """8 heads of 40 is the moonshine streaming encoder's head (hidden 320);
    heads narrower than 64 are stored in zero-padded 64-element ring rows."""
    S, L, T, H = 2, 2, 300, 8
    f = max(right - 1, 0)
    desc = vrt.lookahead_desc(left, right, dtype=dtype, n_layers=L, heads=H, head_dim=d)
    q, k, v = seqs(90 + right, S, L, T, H, d, 1.0, dtype)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    starts = [3, 2 ** 31 - T]   # the second stream ends at the largest position accepted
    runs = {}
    for sizes in ([4], [1], [7], [64], [512]):
        pool = Pool(desc, S, starts)
        say(f"lookahead ({left}, {right}), {H} x {d}: feeds {sizes}")
        runs[sizes[0]] = _feed_all(pool, range(S), L, qd, kd, vd, sizes)
        for s in range(S):
            assert pool.states[s].query(0) == (starts[s], T)
        pool.close()
    base = runs[4]
    assert base.shape[2] == T - f
    for key, out in runs.items():
        assert np.array_equal(out, base), key
    for s in range(S):
        for l in range(L):
            sb = vrt.offline_scratch_bytes(desc, T)
            scratch = torch.empty(sb, dtype=torch.uint8, device=DEV)
            off = torch.empty_like(qd[s, l])
            vrt.enc_attn_offline(desc, qd[s, l], kd[s, l], vd[s, l], T, starts[s], off, scratch, sb, stream())
            torch.cuda.synchronize()
            off = host(off)
            assert np.array_equal(off[:T - f], base[s, l]), (s, l)
            ref = attention.lookahead(q[s, l], k[s, l], v[s, l], left, right)
            check_close(off, ref, dtype, f"stream {s} layer {l}, all {T} rows (offline)")


def test_waiting_counts_must_agree():
    desc = vrt.lookahead_desc(16, 4, n_layers=1)
    q, k, v = seqs(95, 2, 1, 8, 8, 64, 1.0, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    pool = Pool(desc, 2, [0, 0])
    one = [pool.states[0]]
    vrt.enc_attn_feed(one, 0, 1, qd[:1, :, :1].contiguous(), kd[:1, :, :1].contiguous(),
                      vd[:1, :, :1].contiguous(), 1, torch.empty_like(qd[:1, :, :1]), stream())
    torch.cuda.synchronize()
    s = vrt.enc_attn_feed(pool.states, 0, 1, qd[:, :, :4].contiguous(), kd[:, :, :4].contiguous(),
                          vd[:, :, :4].contiguous(), 4, torch.empty_like(qd[:, :, :4]), stream(), check=False)
    assert s == vrt.ERR_INVALID
    assert pool.states[0].query(0) == (0, 1) and pool.states[1].query(0) == (0, 0)
    pool.close()
