"""Pins for the oracle's windowed attention (oracle/attention.py).

* brute force with an explicit T x T mask matrix and pure-Python loops;
* W >= T reduces to plain causal attention: torch's CPU SDPA in float64;
* closed forms: W = 1 gives out = v exactly, q = 0 gives the window mean of v;
* window edge: changing the key/value at p - W leaves out_p bit-identical,
  changing p - W + 1 changes it;
* GQA equals MHA with each kv head repeated Hq/Hkv times;
* shifting every position by the same c leaves the output unchanged."""
import numpy as np
import pytest
import torch

from oracle import attention, rope

THETA = 1.0e6


def _rand(seed, T, hq, hkv, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, hq, d)), rng.standard_normal((T, hkv, d)),
            rng.standard_normal((T, hkv, d)))


@pytest.mark.parametrize("T,W,hq,hkv,d,start", [
    (9, 1, 1, 1, 2, 0), (12, 2, 2, 1, 4, 3), (16, 3, 2, 2, 8, 100),
    (13, 5, 4, 2, 4, 999_990), (7, 16, 1, 1, 8, 0)])
def test_bruteforce_fullmask(T, W, hq, hkv, d, start):
    q, k, v = _rand(T * 7 + W, T, hq, hkv, d)
    a = attention.windowed(q, k, v, start, W, THETA)
    pos = list(range(start, start + T))
    b = attention.windowed_fullmask(q, k, v, pos, W, THETA)
    assert np.max(np.abs(a - b)) <= 1e-13


@pytest.mark.parametrize("d", [8, 64])
def test_large_window_is_causal_sdpa(d):
    T, H = 40, 3
    q, k, v = _rand(d, T, H, H, d)
    start = 17
    out = attention.windowed(q, k, v, start, window=T + 5, theta=THETA)
    pos = np.arange(start, start + T)
    qr = torch.from_numpy(rope.apply(q, pos, THETA)).permute(1, 0, 2)
    kr = torch.from_numpy(rope.apply(k, pos, THETA)).permute(1, 0, 2)
    vv = torch.from_numpy(v).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, is_causal=True)
    ref = ref.permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_window_one_is_identity_on_v():
    q, k, v = _rand(5, 20, 2, 2, 8)
    out = attention.windowed(q, k, v, 0, 1, THETA)
    assert np.array_equal(out, v)


def test_zero_query_is_window_mean():
    T, W = 30, 7
    _, k, v = _rand(6, T, 2, 2, 4)
    q = np.zeros((T, 2, 4))
    out = attention.windowed(q, k, v, 5, W, THETA)
    for t in range(T):
        lo = max(0, t - W + 1)
        assert np.max(np.abs(out[t] - v[lo:t + 1].mean(axis=0))) <= 1e-14


def test_window_edge_perturbation():
    T, W = 24, 6
    q, k, v = _rand(8, T, 2, 2, 8)
    base = attention.windowed(q, k, v, 0, W, THETA)
    t = 15
    # key at position t - W is outside the window of query t
    k2, v2 = k.copy(), v.copy()
    k2[t - W] += 3.0
    v2[t - W] -= 2.0
    out2 = attention.windowed(q, k2, v2, 0, W, THETA)
    assert np.array_equal(out2[t], base[t])
    # key at position t - W + 1 is inside it
    k3 = k.copy()
    k3[t - W + 1] += 3.0
    out3 = attention.windowed(q, k3, v, 0, W, THETA)
    assert not np.array_equal(out3[t], base[t])
    # future keys never matter
    k4, v4 = k.copy(), v.copy()
    k4[t + 1:] = 0.0
    v4[t + 1:] = 1e6
    out4 = attention.windowed(q, k4, v4, 0, W, THETA)
    assert np.array_equal(out4[:t + 1], base[:t + 1])


def test_gqa_equals_repeated_mha():
    T, W, hq, hkv, d = 20, 6, 8, 2, 8
    q, k, v = _rand(9, T, hq, hkv, d)
    g = attention.windowed(q, k, v, 3, W, THETA)
    rep = hq // hkv
    m = attention.windowed(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), 3, W, THETA)
    assert np.max(np.abs(g - m)) <= 1e-13
    # and the mapping is h // rep, not h % hkv: make kv head 1 different
    k_alt = k.copy()
    k_alt[:, 1] *= -1
    g2 = attention.windowed(q, k_alt, v, 3, W, THETA)
    assert np.array_equal(g2[:, :rep], g[:, :rep])
    assert not np.allclose(g2[:, rep:], g[:, rep:])


def test_position_shift_invariance():
    q, k, v = _rand(10, 30, 2, 2, 64)
    a = attention.windowed(q, k, v, 0, 9, THETA)
    b = attention.windowed(q, k, v, 987_654, 9, THETA)
    assert np.max(np.abs(a - b)) <= 1e-9


def test_sampled_rows_equal_whole_sequence():
    T, W = 50, 7
    q, k, v = _rand(11, T, 4, 2, 8)
    full = attention.windowed(q, k, v, 300, W, THETA)
    ts = [0, 1, 6, 7, 30, 49]
    part = attention.windowed_at(q, k, v, 300, W, THETA, ts)
    assert np.array_equal(part, full[ts])


# ---- (left, right) lookahead windows without rotation (moonshine pattern)

def _masked_sdpa(q, k, v, mask):
    """float64 torch SDPA with an explicit boolean mask (True = visible)."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
    return o.numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("T,left,right", [(20, 16, 4), (20, 16, 0), (9, 3, 2), (12, 1, 1), (7, 30, 30)])
def test_lookahead_against_masked_sdpa(T, left, right):
    q, k, v = _rand(T + left + right, T, 2, 2, 8)
    mask = attention.lookahead_mask(T, left, right)
    got = attention.lookahead(q, k, v, left, right)
    ref = _masked_sdpa(q, k, v, mask)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_lookahead_special_cases():
    q, k, v = _rand(5, 10, 2, 2, 4)
    assert np.array_equal(attention.lookahead(q, k, v, 1, 0), v)          # self only
    assert np.array_equal(attention.lookahead(q, k, v, 1, 1), v)          # right = 1: no future
    full = attention.lookahead(q, k, v, 100, 100)                         # whole sequence
    ref = _masked_sdpa(q, k, v, np.ones((10, 10), dtype=bool))
    assert np.max(np.abs(full - ref)) <= 1e-12
    # the page's (16, 4): frame 5 sees frames 0 .. 8
    m = attention.lookahead_mask(20, 16, 4)
    assert list(np.nonzero(m[5])[0]) == list(range(0, 9))
    assert list(np.nonzero(m[19])[0]) == list(range(4, 20))
