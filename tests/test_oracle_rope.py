"""Pins of the oracle's RoPE rotation against mathematics it must satisfy.

Each test checks the oracle against something other than itself: mpmath at
50 digits, the complex-exponential statement of RoPE, the textbook plane
rotation, and the closure/inverse/norm identities (Leyline §2.2).  The negative
controls plant mistakes in copies of the oracle and check that the key
tolerance catches them.
"""

import mpmath
import numpy as np
import pytest

from oracle import bf16, rope, tolerance

mpmath.mp.dps = 50

SHIFTS = [0, 1, -1, -784, 30000, -30000, -60000, 40704, 100000, -100000]
LAYOUTS = [(64, 10000.0), (128, 500000.0)]


@pytest.mark.parametrize("dim,base", LAYOUTS)
def test_inv_freq_matches_mpmath(dim, base):
    th = rope.inv_freq(dim, base)
    for j in range(dim // 2):
        exact = mpmath.power(mpmath.mpf(base), mpmath.mpf(-2 * j) / dim)
        assert abs(th[j] - float(exact)) <= 4e-16 * float(exact)


@pytest.mark.parametrize("dim,base", LAYOUTS)
def test_angles_match_mpmath(dim, base):
    th = rope.inv_freq(dim, base)
    for p in SHIFTS + [62047, 4095 - 784]:
        c, s = rope.cos_sin(p, th)
        for j in range(dim // 2):
            phi = mpmath.mpf(p) * mpmath.power(mpmath.mpf(base), mpmath.mpf(-2 * j) / dim)
            assert abs(c[j] - float(mpmath.cos(phi))) <= 1e-10
            assert abs(s[j] - float(mpmath.sin(phi))) <= 1e-10


@pytest.mark.parametrize("dim,base", LAYOUTS)
def test_rotation_is_complex_exponential(dim, base):
    """RoPE as multiplication of z_j = x_j + i x_{j+h} by exp(i p theta_j)."""
    r = np.random.default_rng(11)
    th = rope.inv_freq(dim, base)
    h = dim // 2
    x = r.standard_normal((50, dim))
    for p in SHIFTS:
        y = rope.rotate(x, p, 1, dim, th)
        z = (x[:, :h] + 1j * x[:, h:]) * np.exp(1j * (p * th))
        scale = np.abs(z) + 1e-300
        assert np.all(np.abs(y[:, :h] - z.real) <= 1e-14 * scale)
        assert np.all(np.abs(y[:, h:] - z.imag) <= 1e-14 * scale)


def test_basis_vectors_are_plane_rotations():
    dim, base = 64, 10000.0
    th = rope.inv_freq(dim, base)
    h = dim // 2
    p = 1234
    for j in (0, 1, 17, h - 1):
        e = np.zeros(dim)
        e[j] = 1.0
        y = rope.rotate(e, p, 1, dim, th)
        expect = np.zeros(dim)
        expect[j] = np.cos(p * th[j])
        expect[j + h] = np.sin(p * th[j])
        assert np.array_equal(y, expect)
        e = np.zeros(dim)
        e[j + h] = 1.0
        y = rope.rotate(e, p, 1, dim, th)
        expect = np.zeros(dim)
        expect[j] = -np.sin(p * th[j])
        expect[j + h] = np.cos(p * th[j])
        assert np.array_equal(y, expect)


@pytest.mark.parametrize("dim,base", LAYOUTS)
def test_closure(dim, base):
    """R(i + D) k == R(D) R(i) k: rotating a stored key equals rotating from scratch.

    The bound is the float64 angle error: each angle p*theta_j (theta_j <= 1)
    is off by at most |p| 2^-52 (product and theta rounding), plus a few ulps
    of cos/sin and of the pair arithmetic.
    """
    r = np.random.default_rng(5)
    th = rope.inv_freq(dim, base)
    k = r.standard_normal((20, dim))
    for i in (0, 7, 1000, 4095, 62047):
        for d in SHIFTS:
            a = rope.rotate(k, i + d, 1, dim, th)
            b = rope.rotate(rope.rotate(k, i, 1, dim, th), d, 1, dim, th)
            bound = ((abs(i) + abs(d) + abs(i + d)) * 2.0 ** -52 + 16 * 2.0 ** -53)
            assert np.max(np.abs(a - b)) <= bound * np.max(np.linalg.norm(k, axis=1))


def test_inverse_and_identity():
    dim, base = 128, 500000.0
    th = rope.inv_freq(dim, base)
    r = np.random.default_rng(2)
    k = r.standard_normal((30, 8 * dim))
    for d in SHIFTS:
        back = rope.rotate(rope.rotate(k, d, 8, dim, th), -d, 8, dim, th)
        assert np.max(np.abs(back - k)) <= 1e-15 * 4 * np.max(np.abs(k))
    assert np.array_equal(rope.rotate(np.abs(k), 0, 8, dim, th), np.abs(k))


def test_pair_norm_preserved():
    dim, base = 64, 10000.0
    th = rope.inv_freq(dim, base)
    r = np.random.default_rng(9)
    k = r.standard_normal((100, dim))
    for d in SHIFTS:
        y = rope.rotate(k, d, 1, dim, th)
        n0 = rope.pair_norms(k, 1, dim)
        n1 = rope.pair_norms(y, 1, dim)
        assert np.max(np.abs(n0 - n1) / n0) <= 1e-15 * 4


def test_heads_rotate_independently():
    dim, base, heads = 128, 500000.0, 8
    th = rope.inv_freq(dim, base)
    r = np.random.default_rng(4)
    k = r.standard_normal((6, heads * dim))
    y = rope.rotate(k, -12345, heads, dim, th)
    for hd in range(heads):
        sl = slice(hd * dim, (hd + 1) * dim)
        assert np.array_equal(y[:, sl], rope.rotate(k[:, sl], -12345, 1, dim, th))


def test_per_row_shifts_broadcast():
    dim, base = 64, 10000.0
    th = rope.inv_freq(dim, base)
    r = np.random.default_rng(8)
    k = r.standard_normal((5, dim))
    p = np.array([3, -9, 0, 100000, -784])
    y = rope.rotate(k, p, 1, dim, th)
    for i in range(5):
        assert np.array_equal(y[i], rope.rotate(k[i], int(p[i]), 1, dim, th))


def test_rotation_against_mpmath_at_large_shift():
    dim, base = 64, 10000.0
    th = rope.inv_freq(dim, base)
    h = dim // 2
    r = np.random.default_rng(12)
    x = r.standard_normal(dim)
    p = 100000
    y = rope.rotate(x, p, 1, dim, th)
    for j in range(h):
        phi = mpmath.mpf(p) * mpmath.power(mpmath.mpf(base), mpmath.mpf(-2 * j) / dim)
        c, s = mpmath.cos(phi), mpmath.sin(phi)
        lo = mpmath.mpf(x[j]) * c - mpmath.mpf(x[j + h]) * s
        hi = mpmath.mpf(x[j]) * s + mpmath.mpf(x[j + h]) * c
        nrm = float(mpmath.sqrt(mpmath.mpf(x[j]) ** 2 + mpmath.mpf(x[j + h]) ** 2))
        assert abs(y[j] - float(lo)) <= 1e-10 * nrm
        assert abs(y[j + h] - float(hi)) <= 1e-10 * nrm


# ------------------------------------------------------- negative controls ---

def _bf16_keys(n, dim, seed):
    r = np.random.default_rng(seed)
    return bf16.round_rne(r.standard_normal((n, dim)))


def _device_like(y):
    """What a correct device returns: fp32 rotation result rounded to bf16."""
    return bf16.round_rne(np.asarray(y, np.float32).astype(np.float64))


@pytest.mark.parametrize("mutant", ["sign", "skip", "swap_pairs", "fp32_angle"])
def test_tolerance_rejects_planted_mistakes(mutant):
    dim, base = 64, 10000.0
    th = rope.inv_freq(dim, base)
    h = dim // 2
    words = _bf16_keys(4000, dim, 21)
    x = bf16.to_f64(words)
    d = 100000 if mutant == "fp32_angle" else -784
    y = rope.rotate(x, d, 1, dim, th)
    norm = rope.pair_norms(x, 1, dim)
    # the correct path passes
    assert tolerance.bf16_close(_device_like(y), y, norm).all()
    if mutant == "sign":
        bad = rope.rotate(x, -d, 1, dim, th)
    elif mutant == "skip":
        bad = x
    elif mutant == "swap_pairs":                      # adjacent pairing instead of half-split
        xs = x.reshape(-1, h, 2)
        c, s = rope.cos_sin(d, th)
        bad = np.stack([xs[..., 0] * c - xs[..., 1] * s, xs[..., 0] * s + xs[..., 1] * c], -1).reshape(x.shape)
    else:                                             # angle formed and reduced in float32
        phi = (np.float32(d) * th.astype(np.float32)).astype(np.float32)
        c = np.cos(phi).astype(np.float64)
        s = np.sin(phi).astype(np.float64)
        bad = np.concatenate([x[:, :h] * c - x[:, h:] * s, x[:, :h] * s + x[:, h:] * c], axis=1)
    ok = tolerance.bf16_close(_device_like(bad), y, norm)
    assert not ok.all()
