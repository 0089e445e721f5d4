"""Helpers for the GPU parity tests: device upload/download, state pools and
the error measures the parity bar is written in.

Tolerances (written in the tests): fp32 storage, norm-wise relative error
max|gpu - oracle| / max|oracle| <= 1e-5 per output tensor; bf16 storage,
max-abs error <= 2e-2 and, since with inputs of scale 0.5 the outputs are
only a few hundredths in size, also the norm-wise relative error
max|gpu - oracle| / max|oracle| <= 1e-2.  The relative bound comes from the
bf16 roundings of the rotated q and k, the softmax weights and the output:
each is an unbiased round-to-nearest-even with relative error at most 2^-9,
the roundings of different keys are independent, so over a window their
effect on an output adds in quadrature and stays a small multiple of 2^-9
(about 2e-3) of the output scale; a wrong key, position or weight moves an
output by a sizeable fraction of it."""
from __future__ import annotations

import sys

import numpy as np
import torch

import sliding_window_cached_amd as vrt
from synth import qkv

DEV = torch.device("cuda:0")
F32_TOL = 1e-5
BF16_TOL = 2e-2
BF16_REL_TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def stream():
    return torch.cuda.current_stream().cuda_stream


def to_dev(x: np.ndarray, dtype: int) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == vrt.BF16 else t


def empty(shape, dtype: int) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == vrt.BF16 else torch.float32,
                       device=DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def rel_err(a, ref) -> float:
    return float(np.abs(np.asarray(a, np.float64) - ref).max() / np.abs(ref).max())


def abs_err(a, ref) -> float:
    return float(np.abs(np.asarray(a, np.float64) - ref).max())


def check_close(a, ref, dtype, what=""):
    if dtype == vrt.F32:
        e = rel_err(a, ref)
        say(f"  {what}: fp32 rel err {e:.3e} (tol {F32_TOL:g})")
        assert e <= F32_TOL, (what, e)
    else:
        e, r = abs_err(a, ref), rel_err(a, ref)
        say(f"  {what}: bf16 max-abs err {e:.3e} (tol {BF16_TOL:g}), rel {r:.3e} "
            f"(tol {BF16_REL_TOL:g})")
        assert e <= BF16_TOL, (what, e)
        assert r <= BF16_REL_TOL, (what, r)


class Pool:
    """n states over one device allocation."""

    def __init__(self, desc, n: int, starts):
        self.desc = desc
        nb = vrt.state_device_bytes(desc)
        self.nbytes = (nb + 255) // 256 * 256      # state memory must be 256-byte aligned
        self.mem = torch.empty(n * self.nbytes, dtype=torch.uint8, device=DEV)
        self.states = [vrt.StreamState(desc, self.mem[i * self.nbytes:(i + 1) * self.nbytes],
                                       nb, int(starts[i])) for i in range(n)]

    def row_elems(self) -> int:
        """Elements per ring row (a lookahead head narrower than 64 is padded)."""
        return max(self.desc.head_dim, 64)

    def ring_rows(self, i: int, layer: int, which: int, head: int, s0: int, s1: int) -> np.ndarray:
        """Rows [s0, s1) of one ring slice, as float32 values."""
        d, r = self.desc, self.row_elems()
        e = 2 if d.dtype == vrt.BF16 else 4
        off = i * self.nbytes + vrt.ring_offset(d, layer, which, head)
        raw = self.mem[off + s0 * r * e: off + s1 * r * e]
        t = raw.view(torch.bfloat16 if e == 2 else torch.float32)
        return t.float().cpu().numpy().reshape(s1 - s0, r)

    def ring_bytes(self, i: int, layer: int, which: int, head: int, s0: int, s1: int) -> bytes:
        d, r = self.desc, self.row_elems()
        e = 2 if d.dtype == vrt.BF16 else 4
        off = i * self.nbytes + vrt.ring_offset(d, layer, which, head)
        return self.mem[off + s0 * r * e: off + s1 * r * e].cpu().numpy().tobytes()

    def close(self):
        for s in self.states:
            s.close()


def run_feeds(pool, idx, layer0, nl, qd, kd, vd, sizes, hooks=None):
    """Feed device sequences [S][nl][T][H][d] in chunks; returns outputs."""
    T = qd.shape[2]
    out = torch.empty_like(qd)
    states = [pool.states[i] for i in idx]
    t, i = 0, 0
    while t < T:
        m = min(sizes[i % len(sizes)], T - t)
        if hooks and i in hooks:
            hooks[i]()
        qc, kc, vc = (x[:, :, t:t + m].contiguous() for x in (qd, kd, vd))
        oc = torch.empty_like(qc)
        vrt.enc_attn_feed(states, layer0, nl, qc, kc, vc, m, oc, stream())
        out[:, :, t:t + m] = oc
        t += m
        i += 1
    torch.cuda.synchronize()
    return out


def seqs(seed, S, L, T, H, d, scale, dtype):
    q = np.empty((S, L, T, H, d), np.float32)
    k, v = np.empty_like(q), np.empty_like(q)
    for s in range(S):
        for l in range(L):
            q[s, l], k[s, l], v[s, l] = qkv(seed, s, l, T, H, H, d, scale,
                                           "bf16" if dtype == vrt.BF16 else "f32")
    return q, k, v
