"""Pins for the streamed oracle (oracle/stream.py): any chunking, with any
compaction points, gives the one-shot result bit for bit; the bounded
re-encode of the last W+n-1 frames gives the same last n outputs bit for bit
(streaming-plan page, bounded-window re-encode section); the decoder's
modulo ring equals a non-wrapping linear buffer (family doc, Streaming row
item 5) and a perturbation of the evicted token cur-8192 changes nothing."""
import numpy as np
import pytest

from oracle import attention
from oracle.stream import EncStream, DecStream
from synth import qkv

THETA = 1.0e6


def _chunks(T, sizes):
    out, t, i = [], 0, 0
    while t < T:
        m = min(sizes[i % len(sizes)], T - t)
        out.append((t, m))
        t += m
        i += 1
    return out


@pytest.mark.parametrize("window,slots,max_batch", [(8, 20, 6), (12, 30, 10)])
@pytest.mark.parametrize("sizes", [[1], [4], [7], [3, 1, 6, 2], [100]])
def test_chunking_is_invisible_small_ring(window, slots, max_batch, sizes):
    T, H, d = 90, 2, 8
    q, k, v = qkv(0, 0, 0, T, H, H, d)
    ref = attention.windowed(q, k, v, 11, window, THETA)
    s = EncStream(H, d, window, slots, max_batch, THETA, start_pos=11)
    out = np.empty_like(ref)
    for t, m in _chunks(T, sizes):
        out[t:t + m] = s.feed(q[t:t + m], k[t:t + m], v[t:t + m])
    assert len(s.ring.events) > 0
    assert np.array_equal(out, ref)


def test_chunking_is_invisible_explicit_compaction():
    # pages' shape: window 8 stands in for 750 at this size; explicit
    # compactions at arbitrary points must not change anything either
    T, H, d = 60, 2, 8
    q, k, v = qkv(1, 0, 0, T, H, H, d)
    ref = attention.windowed(q, k, v, 0, 8, THETA)
    s = EncStream(H, d, 8, 24, 8, THETA)
    out = np.empty_like(ref)
    for i, (t, m) in enumerate(_chunks(T, [4])):
        if i in (3, 4, 9):
            s.compact()
        out[t:t + m] = s.feed(q[t:t + m], k[t:t + m], v[t:t + m])
    assert np.array_equal(out, ref)


@pytest.mark.slow
def test_chunking_is_invisible_full_ring():
    # the real ring (750 / 1536 / 512) with multiple compactions, small H, d
    T, H, d = 2400, 1, 4
    q, k, v = qkv(2, 0, 0, T, H, H, d)
    ref = attention.windowed(q, k, v, 5, 750, THETA)
    for sizes in ([4], [512], [37, 600, 3]):
        s = EncStream(H, d, start_pos=5)
        out = np.empty_like(ref)
        for t, m in _chunks(T, sizes):
            out[t:t + m] = s.feed(q[t:t + m], k[t:t + m], v[t:t + m])
        assert len(s.ring.events) >= 2
        assert np.array_equal(out, ref)


def test_bounded_reencode_equals_full():
    T, W, n = 70, 9, 4
    q, k, v = qkv(3, 0, 0, T, 2, 2, 8)
    full = attention.windowed(q, k, v, 100, W, THETA)
    lo = T - (W + n - 1)
    part = attention.windowed(q[lo:], k[lo:], v[lo:], 100 + lo, W, THETA)
    assert np.array_equal(part[-n:], full[-n:])


def test_decoder_ring_equals_linear_and_oneshot():
    hq, hkv, d, W = 4, 2, 8, 16
    T = 53
    q, k, v = qkv(4, 0, 0, T, hq, hkv, d)
    ref = attention.windowed(q, k, v, 0, W, THETA)
    ring = DecStream(hq, hkv, d, W, W, THETA)
    lin = DecStream(hq, hkv, d, W, 4 * W, THETA)
    a = np.concatenate([ring.step(q[:5], k[:5], v[:5])] +
                       [ring.step(q[t:t + 1], k[t:t + 1], v[t:t + 1]) for t in range(5, T)])
    b = np.concatenate([lin.step(q[:5], k[:5], v[:5])] +
                       [lin.step(q[t:t + 1], k[t:t + 1], v[t:t + 1]) for t in range(5, T)])
    assert np.array_equal(a, b)
    assert np.array_equal(a, ref)


def test_decoder_evicted_token_is_invisible():
    hq, hkv, d, W = 4, 2, 8, 16
    T = 40
    q, k, v = qkv(5, 0, 0, T, hq, hkv, d)
    cur = T - 1
    k2, v2 = k.copy(), v.copy()
    k2[cur - W] += 5.0
    v2[cur - W] += 5.0
    a = attention.windowed(q, k, v, 0, W, THETA)[cur]
    b = attention.windowed(q, k2, v2, 0, W, THETA)[cur]
    assert np.array_equal(a, b)
    k3 = k.copy()
    k3[cur - W + 1] += 5.0
    c = attention.windowed(q, k3, v, 0, W, THETA)[cur]
    assert not np.array_equal(a, c)
