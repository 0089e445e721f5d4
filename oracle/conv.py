"""The causal conv stem ahead of the encoder, offline and streamed, fp64.

TEST INFRASTRUCTURE ONLY (see the package header).

Family doc, "Architecture (summary)", Encoder bullet: a causal left-padded
conv stem, 128 -> 1280 with kernel 3 and stride 1, then 1280 -> 1280 with
kernel 3 and stride 2, each followed by GELU.  Streaming-plan page, "Chunk
alignment": the left padding is (kernel - 1) * dilation + 1 - stride, so 2
for conv0 and 1 for conv1; a streamed conv0 keeps the last 2 input frames as
its padding cache and conv1 the conv0 frames its next output still needs, so
the streamed stem equals the offline one (the offline left padding is the
streamed cache initialised to zeros).

    conv(x)[t][o] = b[o] + sum_k sum_c W[o][c][k] * xpad[t * stride + k][c]
    xpad = (left_pad zero frames) followed by x;  T_out = (T + left_pad - k) // stride + 1
    gelu(x) = x / 2 * (1 + erf(x / sqrt(2)))    (the exact, erf-based GELU)

Weights are [out][in][kernel] as a conv layer stores them.  Reading where the
pages are silent: GELU is the exact erf form.
"""
from __future__ import annotations

import math

import numpy as np

K = 3
PAD0, PAD1 = 2, 1          # (K - 1) + 1 - stride
STRIDE0, STRIDE1 = 1, 2


def left_pad(kernel: int, stride: int, dilation: int = 1) -> int:
    return (kernel - 1) * dilation + 1 - stride


def gelu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def conv_causal(x, W, b, stride: int, pad: int) -> np.ndarray:
    """x [T][C_in], W [C_out][C_in][k], b [C_out] -> [T_out][C_out]."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    T, cin = x.shape
    k = W.shape[2]
    xp = np.concatenate([np.zeros((pad, cin)), x], axis=0)
    n_out = (T + pad - k) // stride + 1 if T + pad >= k else 0
    out = np.empty((n_out, W.shape[0]))
    for t in range(n_out):
        win = xp[t * stride:t * stride + k]          # [k][C_in]
        out[t] = np.einsum("ock,kc->o", W, win) + np.asarray(b, dtype=np.float64)
    return out


def stem(mel, w: dict) -> np.ndarray:
    """Offline stem: gelu(conv1(gelu(conv0(mel))))."""
    h0 = gelu(conv_causal(mel, w["w0"], w["b0"], STRIDE0, PAD0))
    return gelu(conv_causal(h0, w["w1"], w["b1"], STRIDE1, PAD1))


class StreamStem:
    """The stem fed chunk by chunk with explicit padding caches.

    conv0 keeps the last PAD0 input frames (zeros before the first chunk);
    conv1 keeps the conv0 frames not yet consumed by its stride-2 windows
    (one zero frame before the first chunk).  Each feed returns the stem
    outputs that became computable."""

    def __init__(self, w: dict):
        self.w = w
        n_mel = np.asarray(w["w0"]).shape[1]
        d = np.asarray(w["w1"]).shape[0]
        self.cache0 = np.zeros((PAD0, n_mel))
        self.pend1 = np.zeros((PAD1, d))

    def feed(self, mel) -> np.ndarray:
        mel = np.asarray(mel, dtype=np.float64)
        x0 = np.concatenate([self.cache0, mel], axis=0)
        h0 = gelu(conv_causal(x0, self.w["w0"], self.w["b0"], STRIDE0, 0))
        self.cache0 = x0[len(x0) - PAD0:]
        x1 = np.concatenate([self.pend1, h0], axis=0)
        out = gelu(conv_causal(x1, self.w["w1"], self.w["b1"], STRIDE1, 0))
        self.pend1 = x1[STRIDE1 * len(out):]
        return out
