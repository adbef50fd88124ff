"""Pins of the oracle's rotary embedding and token positions.

The pages fix that RoPE is applied to phi(q) and phi(k) right after the ReLU and
that SANA-WM uses a 3-D (t, h, w) rotary embedding; pairing, frequencies and
section order are a documented convention (parity unpinned by the pages).  These
tests pin the convention's internal consistency and its textbook special cases.
"""

import numpy as np
import pytest

import oracle

SPLIT = (8, 12, 12)
BASE = 10000.0


def rand_pos(rng, n, hi=300):
    return tuple(rng.integers(0, hi, n) for _ in range(3))


def test_norm_preserving():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 32))
    y = oracle.rope_rotate(x, *rand_pos(rng, 50), SPLIT, BASE)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def test_identity_at_position_zero():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 32))
    z = np.zeros(7, dtype=np.int64)
    assert np.array_equal(oracle.rope_rotate(x, z, z, z, SPLIT, BASE), x)


def test_relative_position_identity():
    """<R_m x, R_n y> == <x, R_(n-m) y> for every section separately and together."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 32))
    y = rng.standard_normal((40, 32))
    m = rand_pos(rng, 40)
    n = rand_pos(rng, 40)
    lhs = np.sum(oracle.rope_rotate(x, *m, SPLIT, BASE) * oracle.rope_rotate(y, *n, SPLIT, BASE), axis=1)
    diff = tuple(b - a for a, b in zip(m, n))
    rhs = np.sum(x * oracle.rope_rotate(y, *diff, SPLIT, BASE), axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_pair_rotation_is_complex_multiplication():
    """Each adjacent pair (x_a, x_b) turns like the complex number x_a + i x_b times e^(i angle).

    Pair 0 of every section turns by exactly one radian per unit of its position
    (base**0 = 1), which pins the sign and the pairing.
    """
    rng = np.random.default_rng(3)
    x = rng.standard_normal((30, 32))
    pt, ph, pw = rand_pos(rng, 30)
    y = oracle.rope_rotate(x, pt, ph, pw, SPLIT, BASE)
    for off, pos in ((0, pt), (8, ph), (20, pw)):
        zx = x[:, off] + 1j * x[:, off + 1]
        zy = y[:, off] + 1j * y[:, off + 1]
        assert np.allclose(zy, zx * np.exp(1j * pos.astype(float)), rtol=1e-12, atol=1e-12)


def test_frequencies_decrease_along_a_section():
    """Later pairs of a section turn more slowly (a geometric ladder from 1 down towards 1/base)."""
    x = np.zeros((1, 32))
    x[0, 0::2] = 1.0
    one = np.ones(1, dtype=np.int64)
    y = oracle.rope_rotate(x, one, one, one, SPLIT, BASE)
    ang = np.arctan2(y[0, 1::2], y[0, 0::2])
    off = 0
    for d_s in SPLIT:
        a = ang[off // 2: (off + d_s) // 2]
        assert a[0] == pytest.approx(1.0)
        assert np.all(np.diff(a) < 0) and np.all(a > 0)
        ratios = a[1:] / a[:-1]
        assert np.allclose(ratios, ratios[0])              # geometric
        assert ratios[0] ** (d_s // 2) == pytest.approx(1.0 / BASE, rel=1e-9)
        off += d_s


def test_1d_equals_3d_with_empty_spatial_sections():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, 32))
    t = rng.integers(0, 500, 20)
    a = oracle.rope_rotate(x, t, rng.integers(0, 9, 20), rng.integers(0, 9, 20), (32, 0, 0), BASE)
    b = oracle.rope_rotate(x, t, np.zeros(20, int), np.zeros(20, int), (32, 0, 0), BASE)
    assert np.array_equal(a, b)


def test_sections_only_touch_their_channels():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((10, 32))
    z = np.zeros(10, dtype=np.int64)
    p = rng.integers(1, 50, 10)
    y = oracle.rope_rotate(x, z, p, z, SPLIT, BASE)       # only the row section moves
    assert np.array_equal(y[:, :8], x[:, :8]) and np.array_equal(y[:, 20:], x[:, 20:])
    assert not np.allclose(y[:, 8:20], x[:, 8:20])


def test_token_positions_raster_order():
    t, row, col = oracle.token_positions(2 * 6, 6, 3, t0=5)
    assert list(t) == [5] * 6 + [6] * 6
    assert list(row) == [0, 0, 0, 1, 1, 1] * 2
    assert list(col) == [0, 1, 2] * 4
    t, row, col = oracle.token_positions(4, 1, 1)
    assert list(t) == [0, 1, 2, 3] and list(row) == [0] * 4 and list(col) == [0] * 4
