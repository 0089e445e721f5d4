"""The same attention computed incrementally, through explicit fp64 rings.

This is the cached mechanism of the streaming-plan page ("SHIPPED" section:
each new group of frames is written at rows [n_kv_before, n_kv_total) and
then reads rows [0, n_kv_total) under the windowed mask; the ring is
compacted and fed in <=512-frame sub-batches), replayed in fp64 on the CPU.
Per query it gathers the ring rows whose absolute positions lie in
(p - W, p], in ascending position, and calls the same per-row routine as the
one-shot oracle, so a streamed run must equal the one-shot run bit for bit
(streaming-plan page, "Verification" item 1; bunsen streaming chapter,
"Chunking must not be observable").  Empty slots are filled with NaN, so a
read outside the window cannot go unnoticed.
"""
from __future__ import annotations

import numpy as np

from . import rope
from .attention import window_rows
from .ring import EncRing, DecRing, split_feed


class EncStream:
    def __init__(self, heads: int, d: int, window: int = 750, slots: int = 1536,
                 max_batch: int = 512, theta: float = 1e6, start_pos: int = 0):
        self.H, self.d, self.theta = heads, d, theta
        self.ring = EncRing(window, slots, max_batch)
        self.ring.reset(start_pos)
        self.K = np.full((slots, heads, d), np.nan)
        self.V = np.full((slots, heads, d), np.nan)

    def reset(self, start_pos: int) -> None:
        self.ring.reset(start_pos)
        self.K[:] = np.nan
        self.V[:] = np.nan

    def compact(self) -> None:
        n_before = self.ring.n_kv
        ev = self.ring.compact()
        if ev is not None:
            src = slice(ev.shift, n_before)
            self.K[:ev.kept] = self.K[src].copy()
            self.V[:ev.kept] = self.V[src].copy()
            self.K[ev.kept:] = np.nan
            self.V[ev.kept:] = np.nan

    def feed(self, q, k, v) -> np.ndarray:
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        n = q.shape[0]
        out = np.empty_like(q)
        W = self.ring.window
        t = 0
        for m in split_feed(n, self.ring.max_batch):
            if self.ring.needs_compaction(m):
                self.compact()
            s0, p0 = self.ring.append(m)
            pos = p0 + np.arange(m, dtype=np.int64)
            self.K[s0:s0 + m] = rope.apply(k[t:t + m], pos, self.theta)
            self.V[s0:s0 + m] = v[t:t + m]
            qr = rope.apply(q[t:t + m], pos, self.theta)
            base = self.ring.abs_base
            for j in range(m):
                p = int(pos[j])
                lo = max(p - W + 1, base) - base        # slot of the oldest visible key
                hi = p - base                           # slot of the query's own key
                out[t + j] = window_rows(qr[j], np.ascontiguousarray(self.K[lo:hi + 1]),
                                         np.ascontiguousarray(self.V[lo:hi + 1]), 1)
            t += m
        return out


class DecStream:
    """Decoder modulo ring; ``slots`` > window gives the non-wrapping linear
    buffer used for the ring-vs-linear check (family doc, Streaming row item
    5: ring 8192 vs a non-wrapping 16384 buffer)."""

    def __init__(self, hq: int, hkv: int, d: int, window: int = 8192, slots: int = 8192,
                 theta: float = 1e6):
        self.hq, self.hkv, self.d, self.W, self.theta = hq, hkv, d, window, theta
        self.ring = DecRing(slots)
        self.K = np.full((slots, hkv, d), np.nan)
        self.V = np.full((slots, hkv, d), np.nan)

    def step(self, q, k, v) -> np.ndarray:
        """n tokens (n = 1: a decode step; n > 1: a prefill)."""
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        n = q.shape[0]
        p0 = self.ring.next_pos
        pos = p0 + np.arange(n, dtype=np.int64)
        written = self.ring.append(n)
        kr = rope.apply(k, pos, self.theta)
        qr = rope.apply(q, pos, self.theta)
        for j, (p, s) in enumerate(written):
            self.K[s] = kr[j]
            self.V[s] = v[j]
        out = np.empty_like(q)
        group = self.hq // self.hkv
        for j in range(n):
            p = int(pos[j])
            ps = np.arange(max(0, p - self.W + 1), p + 1, dtype=np.int64)
            slots = ps % self.ring.slots
            out[j] = window_rows(qr[j], np.ascontiguousarray(self.K[slots]),
                                 np.ascontiguousarray(self.V[slots]), group)
        return out
