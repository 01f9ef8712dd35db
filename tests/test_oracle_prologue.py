"""Pins of the fp64 QK-norm + rotary oracle (no GPU).

Every pin checks the oracle against something other than its own formula: norms
and angles the rotation must keep, the relative-position property the pages
attribute to rotary embeddings, complex multiplication by a unit phasor (Python's
cmath), finite differences for the backward, and the scale invariance of a
weightless norm.
"""

import cmath
import math

import numpy as np
import pytest

from oracle import prologue as pro


def _x(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("D", [2, 8, 64, 128])
def test_output_has_unit_rms(D):
    """A weightless RMS norm gives unit RMS; the rotation keeps the norm (eps = 0)."""
    y = pro.qk_norm_rope(_x((2, 9, 3, D), D), pos0=[0, 100], eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, atol=1e-12)


def test_position_zero_is_the_norm_alone():
    x = _x((1, 1, 4, 64), 1)
    y = pro.qk_norm_rope(x, eps=1e-6)
    n = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6)
    assert np.array_equal(y, n)


@pytest.mark.parametrize("p", [1, 7, 1000])
def test_pair_rotation_is_a_complex_phasor(p):
    """Pair i of the token at position p turns by p * 10000^(-2i/D): compared, for
    the first and last pair, with multiplication by cmath.exp(1j * angle)."""
    D = 16
    x = _x((1, p + 1, 1, D), p)
    y = pro.qk_norm_rope(x, eps=0.0)[0, p, 0]
    n = x[0, p, 0] / math.sqrt(float(np.mean(x[0, p, 0] ** 2)))
    for i, freq in ((0, 1.0), (D // 2 - 1, 10000.0 ** (-(D - 2) / D))):
        z = complex(n[i], n[i + D // 2]) * cmath.exp(1j * p * freq)
        assert abs(y[i] - z.real) < 1e-12 and abs(y[i + D // 2] - z.imag) < 1e-12


def test_scores_depend_on_relative_position_only():
    """q at position m and k at position n: q'.k' is unchanged when both move by s."""
    D = 64
    q = _x((1, 1, 1, D), 2)
    k = _x((1, 1, 1, D), 3)
    dots = []
    for m, n in ((10, 3), (17, 10), (1010, 1003), (7, 0)):
        yq = pro.qk_norm_rope(q, pos0=m)[0, 0, 0]
        yk = pro.qk_norm_rope(k, pos0=n)[0, 0, 0]
        dots.append(float(yq @ yk))
    assert np.allclose(dots, dots[0], atol=1e-10)
    # and a different offset gives a different score
    yq = pro.qk_norm_rope(q, pos0=12)[0, 0, 0]
    yk = pro.qk_norm_rope(k, pos0=3)[0, 0, 0]
    assert abs(float(yq @ yk) - dots[0]) > 1e-3


def test_norm_and_rotation_commute():
    x = _x((2, 5, 2, 32), 4)
    ang = pro.rope_angles(np.arange(5) + 40, 32).reshape(1, 5, 1, 16)
    a = pro.rotate(pro.rms_norm(x, 0.0), ang)
    b = pro.rms_norm(pro.rotate(x, ang), 0.0)
    assert np.allclose(a, b, atol=1e-13)
    assert np.allclose(pro.qk_norm_rope(x, pos0=40, eps=0.0), a, atol=0)


def test_sequence_offset_shifts_positions():
    """Rows of a sequence with offset o are rows o + t of the same rows placed from 0."""
    x = _x((1, 6, 2, 16), 5)
    pad = np.concatenate([_x((1, 4, 2, 16), 6), x], axis=1)
    assert np.allclose(pro.qk_norm_rope(x, pos0=4), pro.qk_norm_rope(pad)[:, 4:], atol=1e-14)
    # per-sequence offsets; a negative one counts as 0
    xx = np.concatenate([x, x], axis=0)
    y = pro.qk_norm_rope(xx, pos0=[4, -3])
    assert np.array_equal(y[0], pro.qk_norm_rope(x, pos0=4)[0])
    assert np.array_equal(y[1], pro.qk_norm_rope(x)[0])


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
@pytest.mark.parametrize("D", [4, 8])
def test_backward_matches_finite_differences(eps, D):
    x = _x((1, 3, 2, D), 7)
    dy = _x(x.shape, 8)
    g = pro.qk_norm_rope_bwd(x, dy, pos0=5, eps=eps)
    h = 1e-6
    num = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        e = np.zeros_like(x)
        e[idx] = h
        fp = np.sum(pro.qk_norm_rope(x + e, pos0=5, eps=eps) * dy)
        fm = np.sum(pro.qk_norm_rope(x - e, pos0=5, eps=eps) * dy)
        num[idx] = (fp - fm) / (2 * h)
    assert np.max(np.abs(g - num)) / np.max(np.abs(num)) < 1e-6


def test_backward_is_orthogonal_to_the_input():
    """With eps = 0 the forward is unchanged by scaling x, so x . dx = 0 per vector."""
    x = _x((2, 7, 3, 64), 9)
    dx = pro.qk_norm_rope_bwd(x, _x(x.shape, 10), pos0=[0, 300], eps=0.0)
    assert np.max(np.abs(np.sum(x * dx, axis=-1))) < 1e-11
