"""Pins for the oracle's rotary embedding at depth (CPU only)."""

import numpy as np

from oracle.rope import rope


def test_depth_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((5, 3, 64))
    assert np.array_equal(rope(x, np.zeros(5), 10000.0), x)


def test_two_dims_is_a_plane_rotation():
    # D = 2: one pair, frequency theta^0 = 1, so position p rotates by p radians
    x = np.array([[[1.0, 0.0]]])
    y = rope(x, np.array([np.pi / 2]), 10000.0)
    assert np.allclose(y[0, 0], [0.0, 1.0], atol=1e-15)
    y = rope(np.array([[[0.3, -0.7]]]), np.array([1.0]), 10000.0)
    c, s = np.cos(1.0), np.sin(1.0)
    assert np.allclose(y[0, 0], [0.3 * c + 0.7 * s, -0.7 * c + 0.3 * s])


def test_frequencies_at_d4():
    # D = 4, theta = 10000: frequencies 1 and 10000^(-1/2) = 0.01
    x = np.zeros((1, 1, 4))
    x[0, 0, 1] = 1.0                          # second pair: dims 1 and 3
    y = rope(x, np.array([100.0]), 10000.0)
    assert np.allclose(y[0, 0], [0, np.cos(1.0), 0, np.sin(1.0)], atol=1e-14)


def test_complex_closed_form():
    rng = np.random.default_rng(1)
    L, H, D = 17, 2, 64
    x = rng.standard_normal((L, H, D))
    pos = rng.integers(0, 40000, size=L).astype(np.float64)
    y = rope(x, pos, 10000.0)
    half = D // 2
    z = x[..., :half] + 1j * x[..., half:]
    freq = np.power(10000.0, -np.arange(0, D, 2) / D)
    w = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    assert np.allclose(y[..., :half], w.real, atol=1e-9)
    assert np.allclose(y[..., half:], w.imag, atol=1e-9)


def test_relative_position_and_norm():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    dots = []
    for a, b in [(5, 2), (105, 102), (20005, 20002)]:
        dots.append(float(np.sum(rope(q, [a], 1e4) * rope(k, [b], 1e4))))
    assert np.allclose(dots, dots[0], rtol=1e-9)
    assert np.isclose(np.linalg.norm(rope(q, [777], 1e4)), np.linalg.norm(q))
