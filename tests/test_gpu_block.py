"""GPU parity of the encoder attention block around the path (RMSNorm, the
q/k/v projections, the cached attention, the output projection and the
residual) against the fp64 oracle (oracle/block.py), through the C ABI.

Bars, from the arithmetic:
* RMSNorm: fp32 arithmetic and one rounding to bf16, so every element is
  within 2^-8 of the oracle's value relative to it (plus 1e-6 absolute);
* projections: fp32 accumulation of exact bf16 products (error below
  2^-16 of sum |a||w| for these K) and one rounding, so every element is
  within 2^-8 |ref| + 2^-16 (sum_k |a_k w_k| + |bias| + |residual|);
* the block: bf16 rounding at five stored intermediates (normed rows, q,
  k, v, attention output) and at the output, so max|gpu - oracle| <=
  1e-2 max|oracle| on the rows checked;
* chunking: the norm and the projections are row-local and the path is
  bit-exact under chunkings that keep its arithmetic path, so feeds of 4
  and 8 frames (vector path), and of 100 and 512 (matrix path), give
  bit-identical blocks."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
import synth
from oracle import block

from gpu_util import DEV, Pool, host, say, stream

pytestmark = pytest.mark.gpu
THETA = 1.0e6
W = 750


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def test_rmsnorm_elementwise():
    for rows, dim in ((1, 1280), (37, 1280), (5, 64), (300, 2048)):
        x = synth.block_input(60, rows, dim, rows, dim)
        w = synth.block_weights(61, 0, dim)["norm_w"]
        xd, wd = bf(x), bf(w)
        y = torch.empty_like(xd)
        vrt.rmsnorm(xd, rows, dim, wd, 1e-5, y, stream())
        torch.cuda.synchronize()
        ref = block.rmsnorm(x, w)
        d = np.abs(host(y) - ref)
        say(f"  rmsnorm {rows}x{dim}: max rel {float((d / (np.abs(ref) + 1e-30)).max()):.2e}")
        assert np.all(d <= 2.0 ** -8 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("M,K,N,bias,res", [(1, 64, 128, True, False), (37, 128, 256, False, True),
                                            (300, 1280, 1280, True, True), (129, 1280, 3840, True, False),
                                            (4000, 128, 1280, True, True), (4000, 128, 1280, True, "odd"),
                                            (20000, 128, 1280, True, True), (1000, 1280, 1280, True, True)])
def test_linear_elementwise(M, K, N, bias, res):
    """res == "odd": out, bias and residual sit one element past an 8-byte
    boundary (the 2-byte stores and loads of the epilogue)."""
    rng = np.random.default_rng(M + K + N)
    a = synth.round_to(rng.standard_normal((M, K)).astype(np.float32), "bf16")
    w = synth.round_to((rng.standard_normal((N, K)) / K ** 0.5).astype(np.float32), "bf16")
    b = synth.round_to(0.1 * rng.standard_normal(N).astype(np.float32), "bf16") if bias else None
    r = synth.round_to(rng.standard_normal((M, N)).astype(np.float32), "bf16") if res else None
    if res == "odd":
        def odd(t):
            buf = torch.empty(t.numel() + 1, dtype=torch.bfloat16, device=DEV)
            buf[1:] = t.reshape(-1)
            return buf[1:].view(t.shape)
        out = odd(torch.zeros((M, N), dtype=torch.bfloat16, device=DEV))
        bd, rd = odd(bf(b)) if bias else None, odd(bf(r))
    else:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        bd, rd = bf(b) if bias else None, bf(r) if res else None
    vrt.linear(bf(a), M, K, bf(w), N, bd, rd, out, stream())
    torch.cuda.synchronize()
    ref = block.linear(a, w, b) + (r if res else 0.0)
    S = np.abs(a).astype(np.float64) @ np.abs(w).astype(np.float64).T + (np.abs(b) if bias else 0.0) \
        + (np.abs(r) if res else 0.0)
    d = np.abs(host(out) - ref)
    say(f"  linear {M}x{K}x{N}: max abs {float(d.max()):.2e}")
    assert np.all(d <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * S)


def _block_run(kind, S, T, starts, sizes, wts, xs):
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=1, kind=kind)
    pool = Pool(desc, S, starts)
    dim = 1280
    wd = {k: bf(v) for k, v in wts.items()}
    w_qkv = torch.cat([wd["wq"], wd["wk"], wd["wv"]], 0).contiguous()
    bw = vrt.block_weights(wd["norm_w"], w_qkv, wd["bq"], wd["bv"], wd["wo"], wd["bo"], block.EPS)
    xd = bf(np.stack(xs))                                    # [S][T][dim]
    out = torch.empty_like(xd)
    t, i = 0, 0
    while t < T:
        m = min(sizes[i % len(sizes)], T - t)
        wsb = vrt.block_workspace_bytes(desc, S * m)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        xc = xd[:, t:t + m].contiguous()
        oc = torch.empty_like(xc)
        vrt.enc_block_feed(pool.states, 0, xc, m, bw, oc, ws, wsb, stream())
        out[:, t:t + m] = oc
        t, i = t + m, i + 1
    torch.cuda.synchronize()
    pool.close()
    return host(out)


def test_block_feeds_oracle_and_chunking():
    """3 streams, 20 x 64 heads, unaligned starts: a 750-frame pre-fill
    (matrix path) then 4-frame feeds (vector path) up to 1700 frames, across
    compactions; sampled rows against the fp64 block oracle; the same with
    8-frame feeds is bit-identical, and so are 100- and 512-frame feeds."""
    S, T, heads, dim = 3, 1700, 20, 1280
    starts = [0, 4321, 987_654]
    wts = synth.block_weights(62, 0, dim)
    xs = [synth.block_input(63, s, 0, T, dim) for s in range(S)]
    say("block: pre-fill 750, then feeds of 4")
    a = _block_run(vrt.ENC_RING, S, T, starts, [750] + [4] * 300, wts, xs)
    say("block: pre-fill 750, then feeds of 8")
    b = _block_run(vrt.ENC_RING, S, T, starts, [750] + [8] * 200, wts, xs)
    assert np.array_equal(a[:, 750:], b[:, 750:])
    assert np.array_equal(a[:, :750], b[:, :750])
    say("block: feeds of 100 vs 512 (matrix path), modulo ring")
    c = _block_run(vrt.ENC_MODRING, S, T, starts, [100], wts, xs)
    e = _block_run(vrt.ENC_MODRING, S, T, starts, [512], wts, xs)
    assert np.array_equal(c, e)
    for s in range(S):
        ref = block.attn_block(xs[s], wts, heads, starts[s], W, THETA)
        ts = [0, 1, 749, 750, 751, 1535, 1536, 1537, 1699]
        for got, what in ((a[s], "4-frame feeds"), (c[s], "100-frame feeds")):
            err = float(np.abs(got[ts] - ref[ts]).max())
            mx = float(np.abs(ref[ts]).max())
            say(f"  stream {s} {what}: max abs {err:.3e}, max |ref| {mx:.2f}")
            assert err <= 1e-2 * mx


def test_block_serving_batch_tile_shapes():
    """256 streams: a 40-frame feed (the q/k/v product on 256 x 128 tiles,
    the output product on 128 x 128) then 4-frame feeds (the serving step:
    128 x 128 and 64 x 128 tiles), bit-identical to the first 3 streams fed
    as their own batch (64 x 64 tiles throughout), and sampled streams
    against the fp64 block oracle."""
    S, T, heads, dim = 256, 48, 20, 1280
    starts = [(s * 7919) % 1_000_000 for s in range(S)]
    wts = synth.block_weights(64, 0, dim)
    xs = [synth.block_input(65, s, 0, T, dim) for s in range(S)]
    sizes = [40, 4, 4]
    say("block: 256 streams, feeds of 40, 4, 4")
    big = _block_run(vrt.ENC_RING, S, T, starts, sizes, wts, xs)
    say("block: the first 3 streams alone")
    small = _block_run(vrt.ENC_RING, 3, T, starts[:3], sizes, wts, xs[:3])
    assert np.array_equal(big[:3], small)
    ts = [0, 1, 39, 40, 43, 44, 47]
    for s in (0, 131, 255):
        ref = block.attn_block(xs[s], wts, heads, starts[s], W, THETA)
        err = float(np.abs(big[s][ts] - ref[ts]).max())
        mx = float(np.abs(ref[ts]).max())
        say(f"  stream {s}: max abs {err:.3e}, max |ref| {mx:.2f}")
        assert err <= 1e-2 * mx
