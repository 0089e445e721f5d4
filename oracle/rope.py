"""NEOX rotary position embedding in fp64, as a materialised rotation.

Source: Voxtral Realtime family doc, "Architecture (summary)": the encoder
uses NEOX RoPE with theta = 1e6 and head_dim 64, the decoder NEOX RoPE with
theta = 1e6 and head_dim 128, at absolute positions (streaming-plan page,
"SHIPPED" section: the windowed mask and positions are absolute).  NEOX
pairs element i with element i + d/2 ("rotate half"); the moonshine forward
map contrasts this with GPT-J's interleaved pairing ("Decoder block pattern",
"Variant Notes").  The pages do not print the frequency formula; the reading
taken here is the standard one, omega_i = theta^(-2i/d) for i < d/2, with the
angle p * omega_i.
"""
from __future__ import annotations

import numpy as np


def freqs(d: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/d), i = 0 .. d/2-1, in fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / np.float64(d))


def rotation(p, d: int, theta: float) -> np.ndarray:
    """The d x d rotation R_p for each position in ``p`` (shape [..., d, d]).

    Block structure: for i < d/2, rows/cols (i, i+d/2) hold the 2-D rotation
    by angle p*omega_i:  [[cos, -sin], [sin, cos]].
    """
    p = np.asarray(p, dtype=np.float64)
    ang = p[..., None] * freqs(d, theta)           # [..., d/2]
    c, s = np.cos(ang), np.sin(ang)
    h = d // 2
    R = np.zeros(p.shape + (d, d), dtype=np.float64)
    idx = np.arange(h)
    R[..., idx, idx] = c
    R[..., idx, idx + h] = -s
    R[..., idx + h, idx] = s
    R[..., idx + h, idx + h] = c
    return R


def apply(x: np.ndarray, positions, theta: float, chunk: int = 256) -> np.ndarray:
    """Rotate x [T][H][d] by R_{positions[t]} for each row t: x'_t = R x_t.

    The matrix-vector product is written as an elementwise product summed
    over the last axis, so every output element is the same fixed-length sum
    whatever T is (the streamed and one-shot oracles rotate a frame
    identically)."""
    x = np.asarray(x, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    T, H, d = x.shape
    out = np.empty_like(x)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        R = rotation(positions[t0:t1], d, theta)          # [t, d, d]
        out[t0:t1] = (R[:, None, :, :] * x[t0:t1, :, None, :]).sum(axis=-1)
    return out
