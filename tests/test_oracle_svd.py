"""Pins of oracle.svd (patch formation): exact recovery of planted low-rank
deficits, Eckart-Young, an independent power iteration, the factor
convention on non-square deficits with a transposition mutant, and the
orbit mean."""

import math

import numpy as np

from oracle import svd


def test_planted_rank_m_is_recovered_exactly():
    r = np.random.default_rng(60)
    T, F, m = 96, 160, 8
    d = r.standard_normal((T, m)) @ r.standard_normal((m, F))
    U, V, s = svd.truncated_factors(d, m)
    assert U.shape == (T, m) and V.shape == (F, m) and s.shape == (m,)
    assert np.abs(svd.patch(U, V) - d).max() <= 1e-10 * np.abs(d).max()
    assert svd.tail_energy(d, m) <= 1e-18 * (d ** 2).sum()


def test_eckart_young_and_factor_convention():
    r = np.random.default_rng(61)
    T, F, m = 80, 120, 5
    d = r.standard_normal((T, F))
    U, V, s = svd.truncated_factors(d, m)
    err = ((d - svd.patch(U, V)) ** 2).sum()
    assert abs(err - svd.tail_energy(d, m)) <= 1e-9 * (d ** 2).sum()
    assert np.abs(V.T @ V - np.eye(m)).max() <= 1e-12          # V orthonormal
    assert np.abs(U - d @ V).max() <= 1e-10                      # U = U_m Sigma_m = Delta V_m
    assert np.allclose(np.linalg.norm(U, axis=0), s)
    # no rank-m matrix of a few random tries does better
    for _ in range(20):
        a, b = r.standard_normal((T, m)), r.standard_normal((F, m))
        x, *_ = np.linalg.lstsq(a, d, rcond=None)          # best patch with column space of a
        assert ((d - a @ x) ** 2).sum() >= err - 1e-9


def test_leading_triplet_against_power_iteration():
    """sigma_1 and u_1 v_1^T from a plain power iteration (pure Python loops)."""
    r = np.random.default_rng(62)
    T, F = 7, 5
    d = r.standard_normal((T, F))
    d[:, 0] *= 4.0                                  # a clear leading direction
    v = [1.0] * F
    for _ in range(500):
        w = [sum(d[t][f] * v[f] for f in range(F)) for t in range(T)]
        v = [sum(d[t][f] * w[t] for t in range(T)) for f in range(F)]
        nv = math.sqrt(sum(x * x for x in v))
        v = [x / nv for x in v]
    u = [sum(d[t][f] * v[f] for f in range(F)) for t in range(T)]     # sigma_1 u_1
    s1 = math.sqrt(sum(x * x for x in u))
    U, V, s = svd.truncated_factors(d, 1)
    assert abs(s[0] - s1) <= 1e-10 * s1
    p = svd.patch(U, V)
    for t in range(T):
        for f in range(F):
            assert abs(p[t, f] - u[t] * v[f]) <= 1e-9 * s1


def test_transposed_factors_are_rejected():
    """On a square deficit both factor orders have the right shapes; the
    transposed patch V U^T differs from U V^T far beyond any tolerance."""
    r = np.random.default_rng(63)
    d = r.standard_normal((64, 64)) + 3.0 * np.outer(r.standard_normal(64), r.standard_normal(64))
    U, V, _ = svd.truncated_factors(d, 4)
    good, bad = svd.patch(U, V), svd.patch(V, U)
    assert np.linalg.norm(bad - good) > 0.5 * np.linalg.norm(good)


def test_orbit_mean():
    r = np.random.default_rng(64)
    base = r.standard_normal((32, 48))
    assert np.abs(svd.orbit_deficit([base, base, base]) - base).max() <= 1e-15 * np.abs(base).max()
    e = r.standard_normal((4, 32, 48))
    assert np.allclose(svd.orbit_deficit(base + e), base + e.mean(axis=0), atol=1e-14)
    # the orbit patch equals the truncated factors of the mean deficit
    U, V, _ = svd.truncated_factors(svd.orbit_deficit(base + e), 3)
    U2, V2, _ = svd.truncated_factors(base + e.mean(axis=0), 3)
    assert np.allclose(svd.patch(U, V), svd.patch(U2, V2), atol=1e-12)
