"""Seeded synthetic inputs shaped like the streaming-encoder workloads.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention method's arithmetic (no RoPE, no masking, no
softmax), so both the fp64 CPU oracle and the HIP path may take their inputs
from it without sharing any of the computation under test.

Seeding: every tensor of every (stream, layer) comes from its own
``numpy.random.SeedSequence([seed, stream, layer, tensor_id])``.  A stream's
whole sequence of frames is drawn once and then sliced into feeds, so the
values a frame gets never depend on how the stream is chunked.

Workload shapes follow the pages: 20 encoder heads of dim 64 (d_model 1280),
window 750, ring 1536, max batch 512, RoPE theta 1e6 (Voxtral Realtime family
doc, "Architecture (summary)", Encoder bullet; streaming-plan page, "SHIPPED"
section, "Unbounded length" paragraph); decoder GQA 32/8 heads of dim 128 with
window 8192 (family doc, Decoder bullet).  Clip lengths come from the frame
counts the pages quote: 4416 frames (whole-earth), ~15300 frames (dots-full),
and 10 259 / 10 269 tokens for the decoder wrap clips (family doc, Capability
Validation table, Streaming row, items 4 and 5).
"""
from __future__ import annotations

import numpy as np

Q, K, V = 0, 1, 2  # tensor ids in the seed sequence

ENC_HEADS, ENC_DIM = 20, 64
ENC_WINDOW, ENC_RING, MAX_BATCH = 750, 1536, 512
DEC_QHEADS, DEC_KVHEADS, DEC_DIM = 32, 8, 128
DEC_WINDOW = 8192
ROPE_THETA = 1.0e6


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); return the
    raw uint16 bit patterns.  Inputs are finite normal draws (no NaN path)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype; return float32 values that
    are exactly representable in that dtype."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_to_f32(bf16_bits(x))
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(seed: int, stream: int, layer: int, tensor_id: int, shape, scale: float = 1.0,
           dtype: str = "f32") -> np.ndarray:
    """N(0,1)*scale draws for one tensor of one (stream, layer), rounded to
    ``dtype`` and returned as float32 (exact values of that dtype)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, stream, layer, tensor_id]))
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    return round_to(x, dtype)


def qkv(seed: int, stream: int, layer: int, T: int, hq: int, hkv: int, d: int,
        scale: float = 1.0, dtype: str = "f32"):
    """q [T][hq][d], k and v [T][hkv][d] for one (stream, layer)."""
    q = normal(seed, stream, layer, Q, (T, hq, d), scale, dtype)
    k = normal(seed, stream, layer, K, (T, hkv, d), scale, dtype)
    v = normal(seed, stream, layer, V, (T, hkv, d), scale, dtype)
    return q, k, v


X = 3  # tensor id of an encoder block's input rows
NORM_W, WQ, WK, WV, WO, BQ, BV, BO = range(10, 18)  # tensor ids of block weights


def block_input(seed: int, stream: int, layer: int, T: int, dim: int, dtype: str = "bf16"):
    """Block input rows x [T][dim], N(0,1)."""
    return normal(seed, stream, layer, X, (T, dim), 1.0, dtype)


def block_weights(seed: int, layer: int, dim: int, dtype: str = "bf16") -> dict:
    """Random weights of one encoder attention block: norm gain 1 + 0.1 N(0,1),
    projection matrices [out][in] N(0, 1/dim) (unit-variance outputs for
    unit-variance inputs), biases 0.1 N(0,1).  Stream index 0x5EED1 keeps the
    draws apart from any stream's activations."""
    s = 0x5EED1
    w = {"norm_w": 1.0 + normal(seed, s, layer, NORM_W, (dim,), 0.1, "f32")}
    w["norm_w"] = round_to(w["norm_w"], dtype)
    for name, tid in (("wq", WQ), ("wk", WK), ("wv", WV), ("wo", WO)):
        w[name] = normal(seed, s, layer, tid, (dim, dim), dim ** -0.5, dtype)
    for name, tid in (("bq", BQ), ("bv", BV), ("bo", BO)):
        w[name] = normal(seed, s, layer, tid, (dim,), 0.1, dtype)
    return w


W0, B0, W1, B1 = range(20, 24)  # tensor ids of conv stem weights


def conv_weights(seed: int, n_mel: int, d_model: int, dtype: str = "bf16") -> dict:
    """Random conv stem weights in conv layout [out][in][kernel 3]: N(0, 1/fan_in)
    matrices, 0.1 N(0,1) biases."""
    s = 0x5EED2
    return {"w0": normal(seed, s, 0, W0, (d_model, n_mel, 3), (3 * n_mel) ** -0.5, dtype),
            "b0": normal(seed, s, 0, B0, (d_model,), 0.1, dtype),
            "w1": normal(seed, s, 0, W1, (d_model, d_model, 3), (3 * d_model) ** -0.5, dtype),
            "b1": normal(seed, s, 0, B1, (d_model,), 0.1, dtype)}


def mel_frames(seed: int, stream: int, T: int, n_mel: int, dtype: str = "bf16") -> np.ndarray:
    """Log-mel-like input rows [T][n_mel], N(0,1)."""
    return normal(seed, stream, 0, X, (T, n_mel), 1.0, dtype)


def offsets(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi) (start offsets, start positions or
    context lengths), from their own seed sequence."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x5EED, lo, hi]))
    return rng.integers(lo, hi, size=n, dtype=np.int64)
