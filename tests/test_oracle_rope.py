"""Pins for the oracle's NEOX RoPE (oracle/rope.py) against properties the
mathematics fixes: a rotation keeps norms, R_0 is the identity, R_a R_b =
R_{a+b}, q.k depends only on the position difference, d = 2 is the plain
planar rotation by angle p (omega_0 = 1), and the NEOX pairing puts a one-hot
e_0 on indices 0 and d/2 only (not 0 and 1 as GPT-J's interleaving would)."""
import math

import numpy as np
import pytest

from oracle import rope

THETA = 1.0e6


def test_freqs_closed_form():
    w = rope.freqs(64, THETA)
    assert w.shape == (32,)
    assert w[0] == 1.0
    assert abs(w[16] - 1e-3) < 1e-18          # theta^(-1/2)
    assert abs(w[8] - 10 ** (-1.5)) < 1e-16   # theta^(-1/4)
    assert np.all(np.diff(w) < 0)
    w128 = rope.freqs(128, THETA)
    assert abs(w128[32] - 1e-3) < 1e-18


def test_d2_is_planar_rotation():
    for p in [0, 1, 2, 7, 123456]:
        R = rope.rotation(p, 2, THETA)
        c, s = math.cos(p), math.sin(p)
        assert np.allclose(R, [[c, -s], [s, c]], atol=1e-15, rtol=0)
        x = rope.apply(np.array([[[1.0, 0.0]]]), [p], THETA)[0, 0]
        assert abs(x[0] - c) < 1e-15 and abs(x[1] - s) < 1e-15


@pytest.mark.parametrize("d", [4, 64, 128])
def test_neox_pairing_one_hot(d):
    e0 = np.zeros((1, 1, d))
    e0[0, 0, 0] = 1.0
    x = rope.apply(e0, [3], THETA)[0, 0]
    nz = np.nonzero(np.abs(x) > 0)[0].tolist()
    assert nz == [0, d // 2]
    assert abs(x[0] - math.cos(3.0)) < 1e-15 and abs(x[d // 2] - math.sin(3.0)) < 1e-15
    # element d/2 rotates back onto element 0 with the opposite sign
    eh = np.zeros((1, 1, d))
    eh[0, 0, d // 2] = 1.0
    y = rope.apply(eh, [3], THETA)[0, 0]
    assert abs(y[0] + math.sin(3.0)) < 1e-15 and abs(y[d // 2] - math.cos(3.0)) < 1e-15


def test_identity_at_zero_and_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 64))
    assert np.array_equal(rope.apply(x, [0] * 5, THETA), x)
    y = rope.apply(x, [1, 10, 1000, 10 ** 5, 10 ** 6 - 1], THETA)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_composition():
    for a, b in [(3, 5), (700, 49), (10 ** 6, 12345)]:
        Ra, Rb, Rab = (rope.rotation(p, 64, THETA) for p in (a, b, a + b))
        assert np.allclose(Ra @ Rb, Rab, atol=1e-9, rtol=0)
        assert np.allclose(Ra.T @ Ra, np.eye(64), atol=1e-14, rtol=0)


def test_relative_position_invariance():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 4, 64))
    k = rng.standard_normal((1, 4, 64))
    for a, b, c in [(10, 3, 7), (749, 0, 10 ** 6), (5, 5, 999_999)]:
        d0 = (rope.apply(q, [a], THETA) * rope.apply(k, [b], THETA)).sum(-1)
        d1 = (rope.apply(q, [a + c], THETA) * rope.apply(k, [b + c], THETA)).sum(-1)
        tol = 1e-12 if c < 1000 else 1e-9
        assert np.allclose(d0, d1, atol=tol, rtol=0)


def test_sign_convention_rotates_counterclockwise():
    # a key one step behind the query: <R_p q, R_{p-1} k> = <q, R_{-1} k>
    d = 2
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[math.cos(1.0), math.sin(1.0)]]])   # k = R_1 e0
    qr = rope.apply(q, [5], THETA)
    kr = rope.apply(k, [4], THETA)
    # R_4 R_1 e0 = R_5 e0 = R_5 q  =>  the dot product is exactly |q|^2 = 1
    assert abs((qr * kr).sum() - 1.0) < 1e-14
