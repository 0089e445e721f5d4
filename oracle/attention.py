"""Windowed-causal multi-head attention over a whole sequence, fp64.

Definition (streaming-plan page, bounded-window re-encode section: encoder
frame i attends only to frames [i-749, i]; family doc, Streaming row item 5:
the decoder step reveals [cur-8191, cur]): with absolute positions P[t], the
query at t sees exactly the keys u with  P[t] - W < P[u] <= P[t].  Scores are
q.k / sqrt(d) (the pages print no scale; 1/sqrt(head_dim) is the standard
reading), softmax with max-subtraction over the visible keys only, output the
softmax-weighted sum of the (unrotated) values.  q and k are rotated by NEOX
RoPE at their absolute positions first (``oracle.rope``).  GQA (family doc,
Decoder bullet: 32 query heads over 8 kv heads): query head h reads kv head
h // (Hq // Hkv).
"""
from __future__ import annotations

import numpy as np

from . import rope


def window_rows(q_rot: np.ndarray, k_win: np.ndarray, v_win: np.ndarray, group: int) -> np.ndarray:
    """Attention of one query row against a gathered window.

    q_rot [Hq][d]; k_win, v_win [n][Hkv][d] in ascending absolute position.
    Every reduction is an elementwise product summed along a contiguous axis,
    so the result depends only on the gathered values, never on where they
    came from (whole sequence or ring slots)."""
    Hq, d = q_rot.shape
    kv = np.arange(Hq) // group
    kh = np.ascontiguousarray(k_win.transpose(1, 0, 2)[kv])     # [Hq][n][d]
    vh = np.ascontiguousarray(v_win.transpose(1, 2, 0)[kv])     # [Hq][d][n]
    s = (kh * q_rot[:, None, :]).sum(axis=-1) / np.sqrt(np.float64(d))  # [Hq][n]
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    a = e / l
    return (vh * a[:, None, :]).sum(axis=-1)                    # [Hq][d]


def windowed(q, k, v, start_pos: int, window: int, theta: float) -> np.ndarray:
    """Offline windowed-causal attention with positions start_pos + t.

    q [T][Hq][d], k and v [T][Hkv][d] (any float dtype; converted exactly to
    fp64).  Returns out [T][Hq][d] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, d = q.shape
    group = Hq // k.shape[1]
    pos = start_pos + np.arange(T, dtype=np.int64)
    qr = rope.apply(q, pos, theta)
    kr = rope.apply(k, pos, theta)
    out = np.empty((T, Hq, d), dtype=np.float64)
    for t in range(T):
        u0 = max(0, t - window + 1)          # first u with P[t]-W < P[u]
        out[t] = window_rows(qr[t], kr[u0:t + 1], v[u0:t + 1], group)
    return out


def windowed_fullmask(q, k, v, positions, window: int, theta: float) -> np.ndarray:
    """Brute-force form: the explicit T x T mask matrix, pure-Python loops.

    For tiny inputs only.  positions may be any increasing int sequence."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    P = [int(x) for x in positions]
    qr = rope.apply(q, P, theta)
    kr = rope.apply(k, P, theta)
    M = [[(P[t] - window < P[u] <= P[t]) for u in range(T)] for t in range(T)]
    out = np.zeros((T, Hq, d), dtype=np.float64)
    scale = 1.0 / np.sqrt(float(d))
    for t in range(T):
        for h in range(Hq):
            g = h // group
            scores = {}
            for u in range(T):
                if M[t][u]:
                    acc = 0.0
                    for i in range(d):
                        acc += qr[t, h, i] * kr[u, g, i]
                    scores[u] = acc * scale
            mx = max(scores.values())
            w = {u: np.exp(s - mx) for u, s in scores.items()}
            z = sum(w.values())
            for i in range(d):
                out[t, h, i] = sum(w[u] * v[u, g, i] for u in w) / z
    return out


def windowed_at(q, k, v, start_pos: int, window: int, theta: float, ts) -> np.ndarray:
    """Outputs of ``windowed`` for the query rows ``ts`` only, each computed
    from its own gathered window (for sampled checks at sizes where the whole
    sequence would take too long).  Returns [len(ts)][Hq][d] in fp64."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    group = q.shape[1] // k.shape[1]
    out = []
    for t in ts:
        t = int(t)
        u0 = max(0, t - window + 1)
        pos = start_pos + np.arange(u0, t + 1, dtype=np.int64)
        kr = rope.apply(np.asarray(k[u0:t + 1], dtype=np.float64), pos, theta)
        qr = rope.apply(np.asarray(q[t:t + 1], dtype=np.float64), pos[-1:], theta)[0]
        out.append(window_rows(qr, kr, np.asarray(v[u0:t + 1], dtype=np.float64), group))
    return np.stack(out)


def lookahead(q, k, v, left: int, right: int) -> np.ndarray:
    """Sliding-window attention with right lookahead and no rotation, over a
    whole sequence (moonshine forward map, "Per-layer sliding-window mask" and
    the streaming encoder's "Encoder attention" note: no RoPE, per-layer
    (left, right) windows).  The query at t sees the keys u with
    t - u in [0, left) or u - t in (0, right): positions t-left+1 .. t+right-1
    clipped to the sequence.  q [T][Hq][d], k and v [T][Hkv][d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, d = q.shape
    group = Hq // k.shape[1]
    out = np.empty((T, Hq, d), dtype=np.float64)
    for t in range(T):
        u0 = max(0, t - left + 1)
        u1 = min(T - 1, t + max(right - 1, 0))
        out[t] = window_rows(q[t], k[u0:u1 + 1], v[u0:u1 + 1], group)
    return out


def lookahead_mask(T: int, left: int, right: int) -> np.ndarray:
    """The page's mask as a T x T boolean matrix, written out entry by entry:
    visible[q][k] = (q - k in [0, left)) or (k - q in (0, right))."""
    m = np.zeros((T, T), dtype=bool)
    for a in range(T):
        for b in range(T):
            m[a, b] = (0 <= a - b < left) or (0 < b - a < right)
    return m

