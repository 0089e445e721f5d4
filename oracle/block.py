"""The attention half of one encoder block around the cached path, fp64.

TEST INFRASTRUCTURE ONLY (see the package header).

Family doc, "Architecture (summary)", Encoder bullet: the encoder is a stack
of pre-norm RMSNorm blocks; its attention has biases on q, v and o and none
on k, NEOX RoPE (theta 1e6, head_dim 64) and the causal sliding window of
750.  With x [T][dim] the block input (dim = heads * head_dim, features in
head-major order):

    y = x / sqrt(mean(x^2) + eps) * w            RMSNorm over the features
    q = y Wq^T + bq,  k = y Wk^T,  v = y Wv^T + bv
    a = windowed attention of (q, k, v) split into heads (oracle.attention)
    h = x + a Wo^T + bo                           residual around the block

Matrices are [out][in] (one row per output feature).  Readings where the
pages are silent: eps = 1e-5; the residual adds the block input x itself.
"""
from __future__ import annotations

import numpy as np

from . import attention

EPS = 1.0e-5


def rmsnorm(x, w, eps: float = EPS) -> np.ndarray:
    """RMSNorm of every row of x [..][dim] with per-feature gain w [dim]."""
    x = np.asarray(x, dtype=np.float64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def linear(y, W, b=None) -> np.ndarray:
    """y [..][in] times W^T (W [out][in]) plus an optional bias [out]."""
    out = np.asarray(y, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
    if b is not None:
        out = out + np.asarray(b, dtype=np.float64)
    return out


def attn_block(x, wts: dict, heads: int, start_pos: int, window: int, theta: float,
               eps: float = EPS) -> np.ndarray:
    """h [T][dim] for a whole sequence x [T][dim] at positions start_pos + t.

    wts holds norm_w [dim], wq, wk, wv, wo [dim][dim], bq, bv, bo [dim]."""
    x = np.asarray(x, dtype=np.float64)
    T, dim = x.shape
    d = dim // heads
    y = rmsnorm(x, wts["norm_w"], eps)
    q = linear(y, wts["wq"], wts["bq"]).reshape(T, heads, d)
    k = linear(y, wts["wk"]).reshape(T, heads, d)
    v = linear(y, wts["wv"], wts["bv"]).reshape(T, heads, d)
    a = attention.windowed(q, k, v, start_pos, window, theta).reshape(T, dim)
    return x + linear(a, wts["wo"], wts["bo"])
