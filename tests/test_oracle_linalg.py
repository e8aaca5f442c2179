"""Pins for the oracle's SVD routines (Jacobi and randomised range finder)."""
import numpy as np
import pytest

from oracle import linalg


def _check_svd(a, u, s, vt, tol=1e-12):
    p = min(a.shape)
    assert u.shape == (a.shape[0], p) and vt.shape == (p, a.shape[1])
    assert np.all(np.diff(s) <= 1e-12 * s[0])
    nz = s > 1e-12 * s[0]
    assert np.allclose(u[:, nz].T @ u[:, nz], np.eye(nz.sum()), atol=tol)
    assert np.allclose(vt @ vt.T, np.eye(p), atol=tol)
    assert np.linalg.norm(u * s @ vt - a) <= tol * np.linalg.norm(a)


@pytest.mark.parametrize("shape", [(96, 64), (64, 96), (65, 33), (128, 128), (7, 200)])
def test_jacobi_matches_lapack(shape):
    rng = np.random.default_rng(sum(shape))
    a = rng.standard_normal(shape)
    u, s, vt = linalg.jacobi_svd(a)
    ref = np.linalg.svd(a, compute_uv=False)          # LAPACK
    assert np.max(np.abs(s - ref)) <= 1e-9 * ref[0]
    _check_svd(a, u, s, vt)


def test_jacobi_rank_deficient_and_sign_convention():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((80, 6)) @ rng.standard_normal((6, 50))   # rank 6
    u, s, vt = linalg.jacobi_svd(a)
    assert np.all(s[6:] <= 1e-10 * s[0])
    assert np.linalg.norm(u * s @ vt - a) <= 1e-12 * np.linalg.norm(a)
    idx = np.argmax(np.abs(vt[:6]), axis=1)
    assert np.all(vt[np.arange(6), idx] > 0)


def _signs_ok(vt, k):
    idx = np.argmax(np.abs(vt[:k]), axis=1)
    return bool(np.all(vt[np.arange(k), idx] > 0))


@pytest.mark.parametrize("shape", [(30, 70), (70, 30)])
def test_sign_convention_holds_for_wide_and_tall(shape):
    """The convention is on the right singular vectors of the matrix given,
    also when it is wider than tall (decomposed through its transpose)."""
    a = np.random.default_rng(6).standard_normal(shape)
    u, s, vt = linalg.jacobi_svd(a)
    assert _signs_ok(vt, min(shape))
    assert np.linalg.norm(u * s @ vt - a) <= 1e-12 * np.linalg.norm(a)


def test_sign_convention_holds_for_the_range_finder():
    """The randomised path returns factors under the same convention (it
    must not depend on the signs the orthonormal bases happened to get)."""
    rng = np.random.default_rng(7)
    a = rng.standard_normal((300, 500)) * np.linspace(5.0, 0.1, 300)[:, None]
    omega = rng.standard_normal((500, 24))
    u, s, vt = linalg.randomized_svd(a, 8, omega, power_iters=3)
    assert _signs_ok(vt, 8)
    # flipping the sign of the test matrix flips the bases, not the result
    u2, s2, vt2 = linalg.randomized_svd(a, 8, -omega, power_iters=3)
    assert np.allclose(vt, vt2, atol=1e-10) and np.allclose(u, u2, atol=1e-10)
    u3, s3, vt3 = linalg.truncated_svd(a, 8, seed=1)
    assert _signs_ok(vt3, 8)


def test_full_rank_reconstruction_of_smoothed_weight():
    """With r = min(K, N), the fp64 factors reproduce the matrix (north-star
    check 'full-rank reconstruction of W')."""
    rng = np.random.default_rng(11)
    w = rng.standard_normal((192, 128)) * 0.02
    w[5] *= 40.0                       # an outlier row as smoothing produces
    u, s, vt = linalg.truncated_svd(w, 128)
    assert np.linalg.norm(w - (u * s) @ vt) <= 1e-12 * np.linalg.norm(w)


def test_eckart_young_residual():
    rng = np.random.default_rng(12)
    a = rng.standard_normal((120, 90))
    u, s, vt = linalg.truncated_svd(a, 10)
    ref = np.linalg.svd(a, compute_uv=False)
    res = np.linalg.norm(a - (u * s) @ vt) ** 2
    assert abs(res - np.sum(ref[10:] ** 2)) <= 1e-9 * np.sum(ref ** 2)


def test_randomized_recovers_planted_spectrum():
    """A matrix with a clear gap after the leading r values: the randomised
    finder returns those singular values to LAPACK precision."""
    rng = np.random.default_rng(13)
    m, n, r = 400, 900, 12
    q1, _ = np.linalg.qr(rng.standard_normal((m, r)))
    q2, _ = np.linalg.qr(rng.standard_normal((n, r)))
    lead = np.linspace(50.0, 20.0, r)
    a = (q1 * lead) @ q2.T + 1e-3 * rng.standard_normal((m, n))
    omega = rng.standard_normal((n, r + 16))
    u, s, vt = linalg.randomized_svd(a, r, omega, power_iters=4)
    uref, ref, _ = np.linalg.svd(a, full_matrices=False)
    assert np.max(np.abs(s - ref[:r]) / ref[:r]) <= 1e-9
    assert np.allclose(u.T @ u, np.eye(r), atol=1e-10)
    # same leading left subspace as LAPACK, and close to the planted one
    # (noise moves it by about |noise| / gap)
    assert np.linalg.norm(uref[:, :r] - u @ (u.T @ uref[:, :r])) <= 1e-8
    assert np.linalg.norm(q1 - u @ (u.T @ q1)) <= 5e-3


def test_randomized_near_optimal_on_flat_spectrum():
    """Without a gap the truncated answer is not unique; the captured energy is
    still within a few percent of the Eckart-Young optimum."""
    rng = np.random.default_rng(14)
    a = rng.standard_normal((300, 700))
    a[:4] *= 25.0
    u, s, vt = linalg.truncated_svd(a, 16, seed=0)
    ref = np.linalg.svd(a, compute_uv=False)
    res = np.linalg.norm(a - (u * s) @ vt) ** 2
    opt = np.sum(ref[16:] ** 2)
    assert opt <= res <= 1.02 * opt
