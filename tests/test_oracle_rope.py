"""Pins of the oracle's output RoPE (oracle/rope.py)."""
import numpy as np

from oracle import rope as R


def test_identity_composition_and_norms():
    rng = np.random.default_rng(71)
    x = rng.standard_normal((5, 64))
    assert np.array_equal(R.rope_rotate(x, 0, 10000.0), x)
    a = R.rope_rotate(R.rope_rotate(x, 37, 10000.0), 1000, 10000.0)
    assert np.allclose(a, R.rope_rotate(x, 1037, 10000.0), atol=1e-9)
    y = R.rope_rotate(x, 123456, 5e5)
    assert np.allclose(x[:, 0::2] ** 2 + x[:, 1::2] ** 2, y[:, 0::2] ** 2 + y[:, 1::2] ** 2)


def test_relative_position_identity_of_the_pages():
    """R(-i) applied to an entry rotated to its absolute position j equals R(j - i)."""
    rng = np.random.default_rng(72)
    e = rng.standard_normal((8, 64))
    for i, j in [(1000, 20), (262143, 5), (7, 7)]:
        lhs = R.rope_rotate(R.rope_rotate(e, j, 10000.0), -i, 10000.0)
        assert np.allclose(lhs, R.rope_rotate(e, j - i, 10000.0), atol=1e-8)


def test_pairs_are_explicit_planar_rotations():
    x = np.zeros(64); x[10], x[11] = 2.0, -1.0            # pair k = 5
    base, pos = 10000.0, 3.0
    th = pos * base ** (-10 / 64)
    rot = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])
    y = R.rope_rotate(x, pos, base)
    assert np.allclose(y[10:12], rot @ x[10:12])
    assert np.count_nonzero(y) == 2


def test_output_rope_touches_only_the_rope_dims():
    rng = np.random.default_rng(73)
    o = rng.standard_normal((3, 4, 512))
    pos = np.array([0, 5, 1 << 20])
    r = R.output_rope(o, pos[:, None], 10000.0)
    assert np.array_equal(r[..., :448], o[..., :448])
    assert np.array_equal(r[0], o[0])                      # position 0
    assert np.allclose(r[2, :, 448:], R.rope_rotate(o[2, :, 448:], -(1 << 20), 10000.0))
