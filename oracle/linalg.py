"""Singular value decomposition for the low-rank branch (oracle; test infrastructure).

The pages say SVDQuant represents the hardest part of each (smoothed) weight
matrix with a small 16-bit low-rank branch (remio.ai page, "SVDQuant moves hard
values out of 4-bit"; donmalab.com page, core-challenge section). The
decomposition taken for that branch is the truncated SVD, which is the best
rank-r approximation in Frobenius norm (Eckart-Young).

* ``jacobi_svd``: one-sided (Hestenes) Jacobi. Pairs of columns are rotated
  until every pair is orthogonal; column norms are then the singular values.
  Pairs are visited in the round-robin (tournament) order, which lets all
  n/2 disjoint rotations of one round be applied together.
* ``randomized_svd``: for the large layers, a randomised range finder with
  power iterations (Halko, Martinsson and Tropp, SIAM Review 2011, algorithms
  4.3/4.4 and 5.1) reduces the matrix to an l x N problem that the Jacobi
  routine then solves exactly. The random test matrix is an input.

Sign convention (the SVD is unique only up to the sign of each singular pair):
the entry of largest magnitude in each right singular vector is made positive.
"""
from __future__ import annotations

import numpy as np


def _round_robin(n: int):
    """Rounds of the round-robin schedule over n (even) players: n-1 rounds,
    each a list of n/2 disjoint pairs, together covering every pair once."""
    players = list(range(n))
    rounds = []
    for _ in range(n - 1):
        half = n // 2
        rounds.append((np.array(players[:half]), np.array(players[::-1][:half])))
        players = [players[0]] + [players[-1]] + players[1:-1]
    return rounds


def jacobi_svd(a: np.ndarray, tol: float = 1e-15, max_sweeps: int = 60):
    """Thin SVD a = U diag(s) Vt of a real matrix, by one-sided Jacobi in fp64.

    Returns U (m x p), s (p, descending), Vt (p x n) with p = min(m, n)."""
    a = np.asarray(a, dtype=np.float64)
    m, n = a.shape
    if m < n:
        # the transpose's right vectors are this matrix's left ones: the
        # sign convention is applied again, to this matrix's right vectors
        u, s, vt = jacobi_svd(a.T, tol, max_sweeps)
        return _fix_signs(vt.T, s, u.T)
    # Columns of a are kept as contiguous rows of At (and of Vt for V).
    At = np.array(a.T, order="C", copy=True)
    Vt = np.eye(n)
    npad = n + (n % 2)
    if npad != n:  # a zero column pads the schedule; it is never rotated in
        At = np.vstack([At, np.zeros((1, m))])
        Vt = np.pad(Vt, ((0, 1), (0, 1)))
    rounds = _round_robin(npad)
    for _ in range(max_sweeps):
        rotated = False
        for I, J in rounds:
            ai, aj = At[I], At[J]
            alpha = np.einsum("ij,ij->i", ai, ai)
            beta = np.einsum("ij,ij->i", aj, aj)
            gamma = np.einsum("ij,ij->i", ai, aj)
            scale = np.sqrt(alpha * beta)
            act = np.abs(gamma) > tol * scale
            if not act.any():
                continue
            rotated = True
            g = np.where(act, gamma, 1.0)
            zeta = (beta - alpha) / (2.0 * g)
            t = np.where(zeta >= 0, 1.0, -1.0) / (np.abs(zeta) + np.sqrt(1.0 + zeta * zeta))
            c = 1.0 / np.sqrt(1.0 + t * t)
            s = c * t
            c = np.where(act, c, 1.0)[:, None]
            s = np.where(act, s, 0.0)[:, None]
            At[I], At[J] = c * ai - s * aj, s * ai + c * aj
            vi, vj = Vt[I], Vt[J]
            Vt[I], Vt[J] = c * vi - s * vj, s * vi + c * vj
        if not rotated:
            break
    A, V = At[:n].T, Vt[:n, :n].T
    sig = np.sqrt(np.einsum("ij,ij->j", A, A))
    order = np.argsort(-sig, kind="stable")
    sig, A, V = sig[order], A[:, order], V[:, order]
    U = np.zeros_like(A)
    nz = sig > 0
    U[:, nz] = A[:, nz] / sig[nz]
    return _fix_signs(U, sig, V.T)


def _fix_signs(U, s, Vt):
    idx = np.argmax(np.abs(Vt), axis=1)
    sgn = np.sign(Vt[np.arange(Vt.shape[0]), idx])
    sgn[sgn == 0] = 1.0
    return U * sgn, s, Vt * sgn[:, None]


def randomized_svd(a: np.ndarray, rank: int, omega: np.ndarray, power_iters: int = 4):
    """Rank-``rank`` SVD of ``a`` (m x n) from the range of a @ omega.

    ``omega`` is the n x l Gaussian test matrix (l >= rank); it is drawn by the
    caller. Orthonormal bases come from QR (a library primitive). The reduced
    l x n matrix Q^T a is decomposed exactly by ``jacobi_svd``."""
    a = np.asarray(a, dtype=np.float64)
    q, _ = np.linalg.qr(a @ omega)
    for _ in range(power_iters):
        z, _ = np.linalg.qr(a.T @ q)
        q, _ = np.linalg.qr(a @ z)
    b = q.T @ a
    ub, s, vt = jacobi_svd(b)
    u = q @ ub
    return _fix_signs(u[:, :rank], s[:rank], vt[:rank])


def truncated_svd(a: np.ndarray, rank: int, seed: int = 0, exact_limit: int = 256,
                  oversample: int = 16, power_iters: int = 4):
    """Leading ``rank`` singular triplets: exact Jacobi when min(m, n) is at
    most ``exact_limit``, else the randomised range finder (oversampling 16,
    4 power iterations) around Jacobi."""
    m, n = a.shape
    if min(m, n) <= exact_limit:
        u, s, vt = jacobi_svd(a)
        return u[:, :rank], s[:rank], vt[:rank]
    rng = np.random.default_rng(seed)
    omega = rng.standard_normal((n, min(rank + oversample, min(m, n))))
    return randomized_svd(a, rank, omega, power_iters)
