"""Pins for the oracle's causal conv stem (oracle/conv.py).

* the left padding formula gives the pages' values (2 for conv0, 1 for conv1);
* one channel in and out: the causal conv equals numpy's convolution of the
  zero-padded signal with the reversed kernel, subsampled by the stride;
* many channels against pure-Python loops;
* GELU: gelu(1) = Phi(1) (the standard normal CDF at 1, a textbook value),
  gelu(x) - gelu(-x) = x exactly, gelu(0) = 0;
* an 8-frame chunk gives 8 conv0 frames and 4 stem outputs (streaming-plan
  page, "Chunk alignment"), leaving one conv0 frame pending;
* streamed = offline for every chunking tried, odd sizes included;
* receptive field: output j reads conv0 frames 2j-1 .. 2j+1, which read mel
  frames 2j-3 .. 2j+1, so mel frame t reaches exactly the outputs j with
  2j - 3 <= t <= 2j + 1."""
import numpy as np
import pytest

from oracle import conv


def _w(rng, n_mel, d):
    return {"w0": rng.standard_normal((d, n_mel, 3)) / (3 * n_mel) ** 0.5, "b0": 0.1 * rng.standard_normal(d),
            "w1": rng.standard_normal((d, d, 3)) / (3 * d) ** 0.5, "b1": 0.1 * rng.standard_normal(d)}


def test_left_pad_values():
    assert conv.left_pad(3, 1) == 2 == conv.PAD0
    assert conv.left_pad(3, 2) == 1 == conv.PAD1


@pytest.mark.parametrize("stride,pad,T", [(1, 2, 11), (2, 1, 11), (2, 1, 12), (1, 0, 7)])
def test_single_channel_is_numpy_convolution(stride, pad, T):
    rng = np.random.default_rng(stride * 10 + T)
    x, w, b = rng.standard_normal(T), rng.standard_normal(3), rng.standard_normal()
    got = conv.conv_causal(x[:, None], w[None, None, :], [b], stride, pad)[:, 0]
    xp = np.concatenate([np.zeros(pad), x])
    ref = np.convolve(xp, w[::-1], mode="valid")[::stride] + b
    assert got.shape == ref.shape
    assert np.max(np.abs(got - ref)) <= 1e-13


def test_multichannel_loops():
    rng = np.random.default_rng(1)
    T, ci, co, stride, pad = 9, 3, 2, 2, 1
    x, W, b = rng.standard_normal((T, ci)), rng.standard_normal((co, ci, 3)), rng.standard_normal(co)
    got = conv.conv_causal(x, W, b, stride, pad)
    n_out = (T + pad - 3) // stride + 1
    assert got.shape == (n_out, co)
    for t in range(n_out):
        for o in range(co):
            s = float(b[o])
            for k in range(3):
                src = t * stride + k - pad
                if src >= 0:
                    s += sum(float(W[o, c, k]) * float(x[src, c]) for c in range(ci))
            assert abs(got[t, o] - s) <= 1e-13


def test_gelu_values():
    assert abs(conv.gelu(1.0) - 0.8413447460685429) <= 1e-15
    assert abs(conv.gelu(-1.0) + 0.15865525393145707) <= 1e-15
    assert conv.gelu(0.0) == 0.0
    x = np.random.default_rng(2).standard_normal(100) * 3
    assert np.max(np.abs(conv.gelu(x) - conv.gelu(-x) - x)) <= 1e-14


def test_chunk_alignment_of_the_pages():
    rng = np.random.default_rng(3)
    w = _w(rng, 8, 16)
    s = conv.StreamStem(w)
    out = s.feed(rng.standard_normal((8, 8)))
    assert out.shape == (4, 16)            # 8 mel frames -> 4 encoder frames
    assert s.pend1.shape == (1, 16) and s.cache0.shape == (2, 8)
    assert conv.stem(rng.standard_normal((8, 8)), w).shape == (4, 16)


@pytest.mark.parametrize("sizes", [[8], [1], [2, 3], [5, 8, 1, 7], [3], [40]])
def test_streamed_equals_offline(sizes):
    rng = np.random.default_rng(len(sizes))
    w = _w(rng, 8, 16)
    mel = rng.standard_normal((41, 8))
    off = conv.stem(mel, w)
    s, outs, t, i = conv.StreamStem(w), [], 0, 0
    while t < len(mel):
        m = min(sizes[i % len(sizes)], len(mel) - t)
        outs.append(s.feed(mel[t:t + m]))
        t, i = t + m, i + 1
    got = np.concatenate(outs)
    assert got.shape == off.shape
    assert np.array_equal(got, off)


def test_receptive_field():
    rng = np.random.default_rng(4)
    w = _w(rng, 8, 16)
    mel = rng.standard_normal((24, 8))
    base = conv.stem(mel, w)
    for t in (0, 5, 6, 13):
        m2 = mel.copy()
        m2[t] += 1.0
        out = conv.stem(m2, w)
        for j in range(len(base)):
            changed = not np.array_equal(out[j], base[j])
            assert changed == (2 * j - 3 <= t <= 2 * j + 1), (t, j)
