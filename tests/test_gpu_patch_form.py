"""Parity of kamera_patch_factors (HIP, through the C ABI) with the fp64
SVD oracle.  What is unique is compared: the patch U V^T and the singular
values (the factors' column signs are free).

Tolerance: the kernels run in float32 with K <= 1024 products, a shifted
CholeskyQR3 and a 32 x 32 Jacobi eigensolver; their rounding moves the
patch by a few 1e-6 of ||Delta||_F (an fp32 simulation of the same steps on
these deficits gives 2.5e-6), and the sketch's own error is below 1e-7 at
this spectrum.  The bar is 2e-5 ||Delta||_F for the patch and 2e-5 sigma_1
for the singular values."""

import numpy as np
import pytest

import kvsynth
from oracle import svd

pytestmark = pytest.mark.gpu

TOL = 2e-5


def _deficits(n, rows, cols, keys, orders=1, energy_dirs=32, noise=1e-3):
    import torch
    shape = (n, orders, rows, cols) if orders > 1 else (n, rows, cols)
    d = torch.empty(shape, dtype=torch.float32, device="cuda")
    return kvsynth.deficit_batch_(d, energy_dirs, 2.0 ** -0.125, noise, *keys)


def _omega(cols, seed=0):
    import torch
    return torch.from_numpy(kvsynth.rng(8, 9, seed).standard_normal((cols, 32), dtype=np.float32)).cuda()


def _run(d, rank, omega):
    import torch
    import rope_rotation_splice_amd as rrs
    U, V, s = rrs.kamera_patch_factors(d, rank, omega)
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    return U.cpu().double().numpy(), V.cpu().double().numpy(), s.cpu().double().numpy()


def _check(delta, U, V, s, rank):
    U0, V0, s0 = svd.truncated_factors(delta, rank)
    p, p0 = U @ V.T, U0 @ V0.T
    nrm = np.linalg.norm(delta)
    assert np.linalg.norm(p - p0) <= TOL * nrm, f"patch error {np.linalg.norm(p - p0) / nrm:.3g}"
    assert np.abs(s - s0).max() <= TOL * s0[0], f"sigma error {np.abs(s - s0).max() / s0[0]:.3g}"
    assert np.abs(V.T @ V - np.eye(rank)).max() <= 1e-5
    return np.linalg.norm(p - p0) / nrm


@pytest.mark.parametrize("rank", [1, 4, 16])
def test_formation_small_non_square(rank):
    d = _deficits(3, 192, 256, (1, rank))
    U, V, s = _run(d, rank, _omega(256))
    assert U.shape == (3, 192, rank) and V.shape == (3, 256, rank) and s.shape == (3, rank)
    for b in range(3):
        _check(d[b].cpu().double().numpy(), U[b], V[b], s[b], rank)


def test_formation_tall_and_wide():
    for rows, cols in [(640, 128), (128, 576)]:
        d = _deficits(2, rows, cols, (2, rows))
        U, V, s = _run(d, 16, _omega(cols, 1))
        for b in range(2):
            _check(d[b].cpu().double().numpy(), U[b], V[b], s[b], 16)


def test_formation_one_pass_widths():
    """Column counts 512, 768 and 1024 with few rows: the one-pass power
    step at each of its slice widths (256 columns are covered above; 128,
    192 and 576 take the two-pass form)."""
    for rows, cols in [(64, 512), (320, 768), (128, 1024)]:
        d = _deficits(2, rows, cols, (6, cols))
        U, V, s = _run(d, 16, _omega(cols, 5))
        for b in range(2):
            _check(d[b].cpu().double().numpy(), U[b], V[b], s[b], 16)


def test_formation_weak_sketch_direction():
    """Deficits whose sketch Delta^T Delta Omega is ill-conditioned (the
    last of these four meets Omega's columns at a singular value of ~1e-2
    of the top-32 subspace): the orthonormalization's second pass then
    sees a genuine direction at a pivot of ~2e-8 of the largest, which must
    be kept, not dropped as dependent."""
    d = _deficits(4, 128, 1024, (6, 1024))
    U, V, s = _run(d, 16, _omega(1024, 5))
    for b in range(4):
        _check(d[b].cpu().double().numpy(), U[b], V[b], s[b], 16)


def test_orbit_patch_of_the_mean_deficit():
    """Four orders per matrix (the chunk's low-rank directions, with
    order-specific noise at 5x the usual level): the factors are those of
    the mean deficit."""
    d = _deficits(3, 256, 256, (3,), orders=4, noise=5e-3)
    U, V, s = _run(d, 16, _omega(256, 2))
    for b in range(3):
        _check(svd.orbit_deficit(d[b].cpu().double().numpy()), U[b], V[b], s[b], 16)


@pytest.mark.parametrize("orders", [2, 3, 7])
def test_orbit_mean_order_counts(orders):
    """Other order counts: the factors are those of the mean deficit."""
    d = _deficits(2, 128, 192, (5, orders), orders=orders, noise=5e-3)
    U, V, s = _run(d, 8, _omega(192, 4))
    for b in range(2):
        _check(svd.orbit_deficit(d[b].cpu().double().numpy()), U[b], V[b], s[b], 8)


def test_planted_low_rank_and_rank_deficient():
    """A planted rank-8 deficit without noise: with m = 8 the patch is the
    deficit itself; with m = 16 the first 8 singular values are recovered,
    the rest are ~0, and nothing is NaN."""
    import torch
    r = kvsynth.rng(8, 4)
    a = r.standard_normal((2, 256, 8))
    bm = r.standard_normal((2, 8, 192))
    dn = (a @ bm / 16.0).astype(np.float32)
    d = torch.from_numpy(dn).cuda()
    U, V, s = _run(d, 8, _omega(192, 3))
    for b in range(2):
        assert np.linalg.norm(U[b] @ V[b].T - dn[b]) <= TOL * np.linalg.norm(dn[b])
    U, V, s = _run(d, 16, _omega(192, 3))
    assert np.isfinite(U).all() and np.isfinite(V).all() and np.isfinite(s).all()
    for b in range(2):
        s0 = np.linalg.svd(dn[b].astype(np.float64), compute_uv=False)
        assert np.abs(s[b][:8] - s0[:8]).max() <= TOL * s0[0]
        assert s[b][8:].max() <= 1e-3 * s0[0]
        assert np.linalg.norm(U[b] @ V[b].T - dn[b]) <= TOL * np.linalg.norm(dn[b])


def test_formation_workload_sampled():
    """The formation workload (32 layers x 16 chunks x 2 tensors = 1024
    deficits of 1024 x 1024, rank 16) in the configuration the benchmark
    times; deficits 0, 511 and 1023 are compared with the oracle, and every
    deficit's patch is checked to be near-optimal (Eckart-Young) on a
    sample of 8."""
    import torch
    w = kvsynth.patch_formation()
    d = torch.empty((w.n, w.rows, w.cols), dtype=torch.float32, device="cuda")
    kvsynth.deficit_batch_(d, w.energy_dirs, w.decay, w.noise, *w.seed_keys, 1)
    U, V, s = _run(d, w.rank, torch.from_numpy(w.omega).cuda())
    for b in (0, 511, 1023):
        _check(d[b].cpu().double().numpy(), U[b], V[b], s[b], w.rank)
    for b in range(3, w.n, w.n // 8):
        delta = d[b].cpu().double().numpy()
        err = ((delta - U[b] @ V[b].T) ** 2).sum()
        assert err <= (1 + 1e-3) * svd.tail_energy(delta, w.rank) + 1e-9 * (delta ** 2).sum()
