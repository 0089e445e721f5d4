"""The window's edges on the GPU, by perturbation (survey pin P4, on the
kernels): the key at absolute position p - W lies outside query p's window
(p - W, p], so changing its K and V rows must leave out_p bit-identical;
changing the key at p - W + 1 must change out_p; and a key after p, fed in
the same sub-batch as p, must leave out_p bit-identical (the causal mask
inside a sub-batch).  The oracle tolerances cannot see a one-key slip on the
matrix path (one key in 750 moves a bf16 output by about 0.1 %), so this
pins the band mask there exactly.  Query positions are chosen so that p and
p - W + 1 fall on and beside the absolute 64-key tile boundaries and the
32-key half-tiles of the matrix path, after a compaction, on the vector path
(fp32 and bf16, 4-frame feeds) and the matrix path (bf16, 512-frame feeds)
(streaming plan, "SHIPPED": queries see the keys in (p - 750, p])."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt

from gpu_util import DEV, Pool, host, run_feeds, say, seqs, stream, to_dev

pytestmark = pytest.mark.gpu
W = 750


def _edge_queries(start, T):
    ps = set()
    for p in range(W, T):
        a = start + p
        first = a - W + 1
        # p or the window's first key on or next to a 64-key tile or a 32-key half-tile boundary
        if a % 64 in (0, 63) or first % 64 in (0, 1, 63) or first % 32 in (0, 31):
            ps.add(p)
    ps = sorted(ps)
    pick = ps[::max(1, len(ps) // 10)][:10]
    return sorted(set(pick + [W, T - 1]))


@pytest.mark.parametrize("dtype, sizes", [(vrt.F32, [4]), (vrt.BF16, [4]), (vrt.BF16, [512])])
def test_window_edges_by_perturbation(dtype, sizes):
    S, L, T, H, d, start = 1, 1, 1600, 20, 64, 1234 + 17
    desc = vrt.enc_desc(dtype=dtype, n_layers=L)
    q, k, v = seqs(130, S, L, T, H, d, 1.0, dtype)
    qd = to_dev(q, dtype)

    def run(kk, vv):
        pool = Pool(desc, S, [start])
        out = host(run_feeds(pool, [0], 0, L, qd, to_dev(kk, dtype), to_dev(vv, dtype), sizes))
        pool.close()
        return out

    base = run(k, v)
    ps = _edge_queries(start, T)
    say(f"{'bf16' if dtype == vrt.BF16 else 'fp32'} feeds {sizes}: queries {ps}")
    for p in ps:
        for e, unchanged in ((p - W, True), (p - W + 1, False), (p + 1, True)):
            if not 0 <= e < T:
                continue
            kk, vv = k.copy(), v.copy()
            kk[0, 0, e] = kk[0, 0, e] * 3.0 + 1.0
            vv[0, 0, e] = vv[0, 0, e] + 8.0
            out = run(kk, vv)
            same = np.array_equal(out[0, 0, p], base[0, 0, p])
            assert same == unchanged, (p, e, unchanged)


def test_decoder_window_edge_by_perturbation():
    """The decoder's window [cur - 8191, cur] past the ring's wrap: after a
    prefill of 8190 tokens and single steps up to 8199, the step at cur must
    be bit-identical when the token at cur - 8192 (evicted from its slot
    already) is changed, and must change when the token at cur - 8191 (the
    oldest one it sees, read across the wrap) is changed (family doc,
    streaming row: the decoder's ring equals a linear buffer)."""
    L, HQ, HK, DD, N0, cur_max = 1, 32, 8, 128, 8190, 8199
    desc = vrt.dec_desc(n_layers=L)
    rng = np.random.default_rng(7)
    n = cur_max + 1
    q = rng.standard_normal((1, L, n, HQ, DD)).astype(np.float32)
    k = rng.standard_normal((1, L, n, HK, DD)).astype(np.float32)
    v = rng.standard_normal((1, L, n, HK, DD)).astype(np.float32)
    ws_bytes = vrt.dec_workspace_bytes(desc, 1, L, 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)

    def run(kk, vv):
        pool = Pool(desc, 1, [0])
        qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, kk, vv))
        outs = {}
        o = torch.empty_like(qd[:, :, :N0])
        vrt.dec_attn_step(pool.states, 0, L, qd[:, :, :N0].contiguous(), kd[:, :, :N0].contiguous(),
                          vd[:, :, :N0].contiguous(), N0, o, None, 0, stream())
        for c in range(N0, n):
            o1 = torch.empty_like(qd[:, :, c:c + 1])
            vrt.dec_attn_step(pool.states, 0, L, qd[:, :, c:c + 1].contiguous(), kd[:, :, c:c + 1].contiguous(),
                              vd[:, :, c:c + 1].contiguous(), 1, o1, ws, ws_bytes, stream())
            outs[c] = o1
        torch.cuda.synchronize()
        res = {c: host(t) for c, t in outs.items()}
        pool.close()
        return res

    base = run(k, v)
    for cur in (8191, 8192, 8195, 8199):
        for e, unchanged in ((cur - 8192, True), (cur - 8191, False)):
            if e < 0:
                continue
            kk, vv = k.copy(), v.copy()
            kk[0, 0, e] = kk[0, 0, e] * 3.0 + 1.0
            vv[0, 0, e] = vv[0, 0, e] + 8.0
            got = run(kk, vv)
            say(f"decoder step at {cur}: token {e} changed -> output {'unchanged' if unchanged else 'changed'} expected")
            assert np.array_equal(got[cur], base[cur]) == unchanged, (cur, e, unchanged)
