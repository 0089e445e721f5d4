"""Pins for the oracle's encoder attention block (oracle/block.py).

* RMSNorm: constant rows give sign(c) * w, scale invariance and unit mean
  square without eps, a zero row stays zero, and pure-Python loops with eps;
* the projection against pure-Python loops (catches a transposed matrix);
* the whole block against a pure-Python-loop composition built on the
  brute-force attention (explicit mask matrix): per-feature loops for the
  norm and every projection, per-head feature slices, q/v/o biases and no k
  bias, and the residual of the block input;
* closed forms: a zero output projection leaves x + bo exactly."""
import math

import numpy as np
import pytest

from oracle import attention, block

THETA = 1.0e6


def test_rmsnorm_constant_rows_and_invariances():
    rng = np.random.default_rng(0)
    w = rng.standard_normal(16)
    for c in (3.0, -0.25, 1e-3):
        y = block.rmsnorm(np.full((1, 16), c), w, eps=0.0)
        assert np.allclose(y[0], math.copysign(1.0, c) * w, rtol=1e-15, atol=0)
    x = rng.standard_normal((5, 16))
    assert np.allclose(block.rmsnorm(7.5 * x, w, eps=0.0), block.rmsnorm(x, w, eps=0.0),
                       rtol=1e-14, atol=0)
    y1 = block.rmsnorm(x, np.ones(16), eps=0.0)
    assert np.allclose((y1 * y1).mean(axis=-1), 1.0, rtol=1e-14)
    assert np.array_equal(block.rmsnorm(np.zeros((2, 16)), w), np.zeros((2, 16)))


def test_rmsnorm_loops_with_eps():
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((3, 6)), rng.standard_normal(6)
    y = block.rmsnorm(x, w, eps=1e-5)
    for r in range(3):
        ms = sum(float(x[r, i]) ** 2 for i in range(6)) / 6
        for i in range(6):
            assert abs(y[r, i] - float(x[r, i]) / math.sqrt(ms + 1e-5) * float(w[i])) <= 1e-14


def test_linear_loops():
    rng = np.random.default_rng(2)
    y, W, b = rng.standard_normal((4, 5)), rng.standard_normal((3, 5)), rng.standard_normal(3)
    out = block.linear(y, W, b)
    for r in range(4):
        for o in range(3):
            ref = sum(float(y[r, i]) * float(W[o, i]) for i in range(5)) + float(b[o])
            assert abs(out[r, o] - ref) <= 1e-13
    assert np.allclose(block.linear(y, W), out - b, rtol=0, atol=1e-14)


def _weights(rng, dim):
    return {"norm_w": 1 + 0.1 * rng.standard_normal(dim),
            "wq": rng.standard_normal((dim, dim)) / dim ** 0.5,
            "wk": rng.standard_normal((dim, dim)) / dim ** 0.5,
            "wv": rng.standard_normal((dim, dim)) / dim ** 0.5,
            "wo": rng.standard_normal((dim, dim)) / dim ** 0.5,
            "bq": 0.1 * rng.standard_normal(dim), "bv": 0.1 * rng.standard_normal(dim),
            "bo": 0.1 * rng.standard_normal(dim)}


def _loops_block(x, wt, heads, start, window):
    T, dim = x.shape
    d = dim // heads
    eps = block.EPS
    y = np.empty((T, dim))
    for t in range(T):
        ms = sum(float(x[t, i]) ** 2 for i in range(dim)) / dim
        for i in range(dim):
            y[t, i] = float(x[t, i]) / math.sqrt(ms + eps) * float(wt["norm_w"][i])

    def proj(W, b):
        out = np.empty((T, dim))
        for t in range(T):
            for o in range(dim):
                out[t, o] = sum(y[t, i] * float(W[o, i]) for i in range(dim)) + (float(b[o]) if b is not None else 0.0)
        return out

    q, k, v = proj(wt["wq"], wt["bq"]), proj(wt["wk"], None), proj(wt["wv"], wt["bv"])
    a = np.empty((T, dim))
    pos = list(range(start, start + T))
    for h in range(heads):   # features h*d .. h*d+d-1 form head h
        sl = slice(h * d, (h + 1) * d)
        a[:, sl] = attention.windowed_fullmask(q[:, None, sl], k[:, None, sl], v[:, None, sl],
                                               pos, window, THETA)[:, 0]
    h_out = np.empty((T, dim))
    for t in range(T):
        for o in range(dim):
            h_out[t, o] = float(x[t, o]) + sum(a[t, i] * float(wt["wo"][o, i]) for i in range(dim)) \
                + float(wt["bo"][o])
    return h_out


@pytest.mark.parametrize("T,heads,d,window,start", [(7, 2, 4, 3, 0), (9, 3, 2, 4, 123_457), (5, 1, 8, 16, 5)])
def test_block_against_loops(T, heads, d, window, start):
    rng = np.random.default_rng(T * 31 + heads)
    dim = heads * d
    x = rng.standard_normal((T, dim))
    wt = _weights(rng, dim)
    got = block.attn_block(x, wt, heads, start, window, THETA)
    ref = _loops_block(x, wt, heads, start, window)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_zero_output_projection():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 8))
    wt = _weights(rng, 8)
    wt["wo"] = np.zeros((8, 8))
    assert np.array_equal(block.attn_block(x, wt, 2, 0, 4, THETA), x + wt["bo"])
