"""Pins for the oracle's RoPE and RMSNorm: closed forms and textbook identities."""

import math

import numpy as np
import pytest

from oracle import rope_neox, rms_norm, qk_transform

D = 128


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((3, D))
    assert np.array_equal(rope_neox(x, 0, 1e4), x)


@pytest.mark.parametrize("i", [0, 1, 17, 63])
@pytest.mark.parametrize("pos", [1, 5, 4095, 131071, 262143])
def test_rope_one_hot_closed_form(i, pos):
    """e_i rotates to cos(a) e_i + sin(a) e_{i+64}; e_{i+64} to -sin(a) e_i + cos(a) e_{i+64},
    with a = pos * 10000**(-2i/128), computed here with the math module."""
    a = pos * 10000.0 ** (-2.0 * i / D)
    x = np.zeros(D)
    x[i] = 1.0
    y = rope_neox(x, pos, 1e4)
    want = np.zeros(D)
    want[i], want[i + 64] = math.cos(a), math.sin(a)
    assert np.allclose(y, want, rtol=0, atol=1e-15)
    x = np.zeros(D)
    x[i + 64] = 1.0
    y = rope_neox(x, pos, 1e4)
    want = np.zeros(D)
    want[i], want[i + 64] = -math.sin(a), math.cos(a)
    assert np.allclose(y, want, rtol=0, atol=1e-15)


def test_rope_equals_complex_rotation():
    """Textbook form: pair (x_i, x_{i+64}) as z = x_i + i x_{i+64}, rotated by e^{i a}."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, D))
    for pos in (3, 1000, 200_000):
        a = pos * np.power(1e4, -2.0 * np.arange(64) / D)
        z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * a)
        want = np.concatenate([z.real, z.imag], axis=1)
        assert np.allclose(rope_neox(x, pos, 1e4), want, rtol=0, atol=1e-12)


def test_rope_preserves_norm_and_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for m, n in [(10, 3), (4096, 17), (131071, 65536)]:
        rq, rk = rope_neox(q, m, 1e4), rope_neox(k, n, 1e4)
        assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) < 1e-12
        assert abs(np.dot(rq, rk) - np.dot(rope_neox(q, m - n, 1e4), k)) < 1e-9


def test_rms_norm_constant_vector_closed_form():
    for c in (0.5, 3.0, -2.0):
        w = np.linspace(0.5, 1.5, D)
        y = rms_norm(np.full(D, c), w, 1e-6)
        assert np.allclose(y, w * c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)


def test_rms_norm_brute_force_and_identities():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(D)
    w = 1 + 0.1 * rng.standard_normal(D)
    eps = 1e-6
    ms = sum(float(v) * float(v) for v in x) / D
    want = [float(x[i]) / math.sqrt(ms + eps) * float(w[i]) for i in range(D)]
    y = rms_norm(x, w, eps)
    assert np.allclose(y, want, rtol=1e-14, atol=0)
    # scale invariance far above eps, and the RMS of y / w
    # relative effect of eps is eps / (2 mean(x^2)) ~ 5e-7 here, and 1e6 times smaller at 1000 x
    assert np.allclose(rms_norm(1000 * x, w, eps), rms_norm(x, w, 0.0), rtol=1e-12)
    assert np.allclose(y, rms_norm(x, w, 0.0), rtol=2 * eps / ms)
    rms = math.sqrt(np.mean((y / w) ** 2))
    assert abs(rms - (1 + eps / ms) ** -0.5) < 1e-14


def test_norm_and_rope_orders_agree_with_unit_weight():
    """The only part of the order question that is pinned (R2)."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, D))
    one = np.ones(D)
    a = qk_transform(x, one, 777, 1e4, 1e-6, norm_before_rope=False)
    b = qk_transform(x, one, 777, 1e4, 1e-6, norm_before_rope=True)
    assert np.allclose(a, b, rtol=0, atol=1e-13)
    # with a non-trivial weight they differ, so the flag does something
    w = 1 + 0.1 * rng.standard_normal(D)
    a = qk_transform(x, w, 777, 1e4, 1e-6, norm_before_rope=False)
    b = qk_transform(x, w, 777, 1e4, 1e-6, norm_before_rope=True)
    assert np.max(np.abs(a - b)) > 1e-3


def _unrotate(y, pos, theta):
    """Inverse of rotate-half RoPE, written as the complex rotation by -angle:
    channel pairs (i, i + D/2) are the real and imaginary parts of z_i."""
    half = D // 2
    a = pos * theta ** (-2.0 * np.arange(half) / D)
    z = (y[..., :half] + 1j * y[..., half:]) * np.exp(-1j * a)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("pos", [0, 1, 777, 131071])
def test_composition_order_invariants(pos):
    """Each order leaves its own trace whatever the weights: with the norm last
    (the default, R2), y / w has RMS sqrt(ms / (ms + eps)) for ms = mean(x^2)
    (RoPE keeps ms); with RoPE last, rotating y back gives a vector whose ratio
    to w has that RMS.  A swapped order, a dropped step or a weight applied in
    the wrong place breaks the one that is asserted."""
    rng = np.random.default_rng(40 + pos % 97)
    x = rng.standard_normal((6, D)) * rng.uniform(0.01, 30.0, (6, 1))
    w = 1 + 0.3 * rng.standard_normal(D)
    eps = 1e-6
    ms = np.mean(x * x, axis=-1)
    want = np.sqrt(ms / (ms + eps))
    y = qk_transform(x, w, pos, 1e4, eps, norm_before_rope=False)
    got = np.sqrt(np.mean((y / w) ** 2, axis=-1))
    assert np.allclose(got, want, rtol=1e-12, atol=0)
    y2 = qk_transform(x, w, pos, 1e4, eps, norm_before_rope=True)
    got2 = np.sqrt(np.mean((_unrotate(y2, pos, 1e4) / w) ** 2, axis=-1))
    assert np.allclose(got2, want, rtol=1e-12, atol=0)
    # and each invariant fails for the other order once the weight is not flat
    if pos:
        assert not np.allclose(np.sqrt(np.mean((y2 / w) ** 2, axis=-1)), want, rtol=1e-6, atol=0)
