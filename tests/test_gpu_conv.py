"""GPU parity of the causal conv stem (two kernel-3 convs on the matrix cores,
strides 1 and 2, bias, exact GELU, padding caches across feeds) against the
fp64 oracle (oracle/conv.py), through the C ABI.

Bars:
* every stem output agrees with the oracle's offline stem within
  1e-2 max|oracle| (bf16 rounding of the conv0 rows and of the outputs;
  fp32 accumulation);
* a stream fed in the pages' 8-frame chunks, in mixed chunk sizes (odd ones
  included, which change how many conv0 frames are carried) and in one
  feed gives bit-identical outputs: every output row's k order is fixed;
* a reset stem equals a fresh one bit for bit."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
import synth
from oracle import conv

from gpu_util import DEV, host, say, stream

pytestmark = pytest.mark.gpu
N_MEL, D = 128, 1280


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def _weights(w):
    tap_major = lambda W: np.ascontiguousarray(np.transpose(W, (0, 2, 1)).reshape(W.shape[0], -1))
    t = {"w0": bf(tap_major(w["w0"])), "b0": bf(w["b0"]), "w1": bf(tap_major(w["w1"])), "b1": bf(w["b1"])}
    return t, vrt.conv_weights(t["w0"], t["b0"], t["w1"], t["b1"])


def _run(S, mel, sizes, cw, stems=None):
    """Feed mel [S][T][n_mel] in chunks; return the concatenated outputs."""
    T = mel.shape[1]
    nb = vrt.conv_stem_device_bytes(N_MEL, D)
    own = stems is None
    if own:
        mem = torch.empty(S * nb, dtype=torch.uint8, device=DEV)
        stems = [vrt.ConvStem(N_MEL, D, mem[i * nb:(i + 1) * nb], nb) for i in range(S)]
    outs, t, i = [], 0, 0
    while t < T:
        m = min(sizes[i % len(sizes)], T - t)
        n_out = stems[0].out_frames(m)
        wsb = vrt.conv_workspace_bytes(N_MEL, D, S, m)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        o = torch.empty((S, max(n_out, 1), D), dtype=torch.bfloat16, device=DEV)
        got = vrt.conv_stem_feed(stems, mel[:, t:t + m].contiguous(), m, cw, o, ws, wsb, stream())
        assert got == n_out
        if n_out:
            outs.append(o[:, :n_out].clone())
        t, i = t + m, i + 1
    torch.cuda.synchronize()
    res = host(torch.cat(outs, dim=1))
    if own:
        for s in stems:
            s.close()
    return res, stems


def test_conv_stem_oracle_and_chunkings():
    S, T = 3, 72
    w = synth.conv_weights(70, N_MEL, D)
    tens, cw = _weights(w)
    mel_np = np.stack([synth.mel_frames(71, s, T, N_MEL) for s in range(S)])
    mel = bf(mel_np)
    say("conv stem: 8-frame chunks")
    a, _ = _run(S, mel, [8], cw)
    say("conv stem: mixed chunks 5, 3, 8, 1, 7, 2")
    b, _ = _run(S, mel, [5, 3, 8, 1, 7, 2], cw)
    say("conv stem: one feed")
    c, _ = _run(S, mel, [T], cw)
    assert a.shape == (S, T // 2, D)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    for s in range(S):
        ref = conv.stem(mel_np[s], w)
        err, mx = float(np.abs(a[s] - ref).max()), float(np.abs(ref).max())
        say(f"  stream {s}: max abs {err:.3e}, max |ref| {mx:.2f}")
        assert err <= 1e-2 * mx


def test_conv_stem_serving_batch_tile_invariance():
    """256 stems x 8 mel frames (the serving step: conv0 2048 rows, conv1
    1024 rows in three k parts, on the large tiles) against the oracle on
    sampled stems, and bit-identical to the same stems fed as a batch of 3
    (the smallest tiles): every tile shape keeps each output's k order."""
    S, T = 256, 8
    w = synth.conv_weights(74, N_MEL, D)
    tens, cw = _weights(w)
    mel_np = np.stack([synth.mel_frames(75, s, T, N_MEL) for s in range(S)])
    mel = bf(mel_np)
    say("conv stem: 256 stems, one 8-frame feed")
    big, _ = _run(S, mel, [T], cw)
    small, _ = _run(3, mel[:3].contiguous(), [T], cw)
    assert np.array_equal(big[:3], small)
    for s in (0, 1, 77, 128, 200, 255):
        ref = conv.stem(mel_np[s], w)
        err, mx = float(np.abs(big[s] - ref).max()), float(np.abs(ref).max())
        say(f"  stream {s}: max abs {err:.3e}, max |ref| {mx:.2f}")
        assert err <= 1e-2 * mx


def test_conv_stem_reset_equals_fresh():
    S, T = 2, 24
    w = synth.conv_weights(72, N_MEL, D)
    tens, cw = _weights(w)
    mel = bf(np.stack([synth.mel_frames(73, s, T, N_MEL) for s in range(S)]))
    nb = vrt.conv_stem_device_bytes(N_MEL, D)
    mem = torch.empty(S * nb, dtype=torch.uint8, device=DEV)
    stems = [vrt.ConvStem(N_MEL, D, mem[i * nb:(i + 1) * nb], nb) for i in range(S)]
    a, _ = _run(S, mel, [8], cw, stems)
    assert stems[0].query() == (T, 1)
    for st in stems:
        st.reset()
    b, _ = _run(S, mel, [7, 9], cw, stems)
    assert np.array_equal(a, b)
    for st in stems:
        st.close()
