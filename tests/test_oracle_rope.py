"""Pins of the oracle's RoPE table and rotations against closed forms."""
import math

import numpy as np
import pytest

from oracle import rope

pytestmark = pytest.mark.cpu


def test_inverse_frequencies():
    th = rope.inv_freq(128, 10000.0)
    assert th[0] == 1.0
    assert th.size == 64
    assert np.allclose(th[1:] / th[:-1], 10000.0 ** (-2.0 / 128), rtol=1e-14)
    assert math.isclose(th[-1], 10000.0 ** (-126.0 / 128), rel_tol=1e-15)


def test_position_zero_is_identity():
    c, s = rope.cos_sin([0], 64)
    assert np.all(c == 1.0) and np.all(s == 0.0)
    x = np.random.default_rng(0).standard_normal((5, 3, 64)).astype(np.float32)
    assert np.array_equal(rope.rotate(x, c[0], s[0]), x)
    assert np.array_equal(rope.rotate_back(x, c[0], s[0]), x)


def test_table_against_an_independent_cos_sin():
    pos = np.array([1, 2, 3, 757, 5788, 6812, 31793, 32767, 65535])
    c, s = rope.cos_sin(pos, 128)
    ang = pos[:, None].astype(np.float64) * rope.inv_freq(128)[None, :]
    cn = np.cos(ang).astype(np.float32)
    sn = np.sin(ang).astype(np.float32)
    # numpy's vectorised cos/sin may differ from libm by one fp64 ulp, which can
    # move the fp32 rounding by at most one fp32 ulp
    assert np.all(np.abs(c.view(np.int32) - cn.view(np.int32)) <= 1)
    assert np.all(np.abs(s.view(np.int32) - sn.view(np.int32)) <= 1)
    assert np.max(np.abs(c.astype(np.float64) - np.cos(ang))) <= 2.0 ** -24
    assert np.max(np.abs(s.astype(np.float64) - np.sin(ang))) <= 2.0 ** -24


def test_rotation_matches_complex_multiplication():
    rng = np.random.default_rng(1)
    d = 128
    pos = np.arange(0, 20000, 997)
    x = rng.standard_normal((pos.size, 2, d)).astype(np.float32)
    c, s = rope.cos_sin(pos, d)
    got = rope.rotate(x, c[:, None, :], s[:, None, :]).astype(np.float64)
    z = (x[..., 0::2].astype(np.float64) + 1j * x[..., 1::2].astype(np.float64))
    w = (c.astype(np.float64) + 1j * s.astype(np.float64))[:, None, :]
    ref = z * w
    mag = np.abs(z)
    assert np.all(np.abs(got[..., 0::2] - ref.real) <= 2.0 ** -22 * mag + 1e-30)
    assert np.all(np.abs(got[..., 1::2] - ref.imag) <= 2.0 ** -22 * mag + 1e-30)
    # and against the ideal angle (table rounding included)
    ideal = rope.rotate64(x.astype(np.float64), pos, d)
    assert np.max(np.abs(got - ideal) / (np.repeat(mag, 2, axis=-1) + 1e-30)) < 2.0 ** -20


def test_rotation_preserves_pair_norm():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 4, 64)).astype(np.float32)
    c, s = rope.cos_sin(np.arange(64) * 37, 64)
    y = rope.rotate(x, c[:, None, :], s[:, None, :]).astype(np.float64)
    n0 = x[..., 0::2].astype(np.float64) ** 2 + x[..., 1::2].astype(np.float64) ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(n1 - n0) / n0) < 1e-6


def test_rotate_back_inverts_rotate():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 2, 64)).astype(np.float32)
    c, s = rope.cos_sin([1234], 64)
    y = rope.rotate_back(rope.rotate(x, c[0], s[0]), c[0], s[0])
    assert np.max(np.abs(y - x)) < 1e-5 * np.max(np.abs(x))


def test_composition_law_fp64():
    """R(a)^T R(b) = R(b - a) for the fp64 rotation, and R(-D) R(p) = R(p - D)."""
    d = 16
    th = rope.inv_freq(d)
    for a, b in [(3, 10), (757, 6812), (31794, 5), (0, 40000)]:
        for i, t in enumerate(th):
            Ra = np.array([[math.cos(a * t), -math.sin(a * t)], [math.sin(a * t), math.cos(a * t)]])
            Rb = np.array([[math.cos(b * t), -math.sin(b * t)], [math.sin(b * t), math.cos(b * t)]])
            Rd = np.array([[math.cos((b - a) * t), -math.sin((b - a) * t)],
                           [math.sin((b - a) * t), math.cos((b - a) * t)]])
            assert np.max(np.abs(Ra.T @ Rb - Rd)) < 1e-11
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 3, d))
    p = np.array([5, 100, 6000, 31793, 40, 0, 12345])
    D = 31794
    y = rope.rotate64(rope.rotate64(x, p, d), np.full(7, -D), d)
    z = rope.rotate64(x, p - D, d)
    assert np.max(np.abs(y - z)) < 1e-11
