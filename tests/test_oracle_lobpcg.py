"""Pins of the oracle's LOBPCG eigensolver (oracle/lobpcg.py) against facts fixed by
the mathematics.

  eigenpairs   numpy.linalg.eigh of the dense matrix (an independent library routine
               on A itself), both ends; the closed-form spectrum of the 5-point
               Laplacian on an Nx x Ny grid; a start block spanning an invariant
               subspace (exact pairs at iteration 0); the reported residuals are the
               true |A u - theta u| and meet the stop test; orthonormal vectors with
               <u_r, X0[r]> >= 0.
  Rayleigh-Ritz  every iteration's basis contains the previous Ritz vectors, so by
               Courant-Fischer the Ritz values move monotonically toward the wanted
               end, and by Cauchy interlacing they never pass the true eigenvalues.
  two methods  the Lanczos oracle (oracle/eigsh.py), a different algorithm, converges
               to the same eigenvalues.
The module under test can be replaced through SLA_ORACLE_LOBPCG (a path to a modified
copy), which tests/test_oracle_mutations.py uses to plant mistakes.
"""
import importlib.util
import math
import os

import numpy as np
import pytest
import scipy.sparse as sp

import oracle as O
import workloads as W


def _load():
    path = os.environ.get("SLA_ORACLE_LOBPCG")
    if not path:
        from oracle import lobpcg as L
        return L
    spec = importlib.util.spec_from_file_location("oracle.lobpcg_under_test", path)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    spec.loader.exec_module(mod)
    return mod


L = _load()


def dense(A):
    return sp.csr_matrix((A.vals, A.col, A.row_ptr.astype(np.int64)), shape=(A.n_rows, A.n_cols)).toarray()


def csr_of_dense(M):
    S = sp.csr_matrix(M)
    S.sort_indices()
    return W.CSR(M.shape[0], M.shape[1], S.indptr.astype(np.int32), S.indices.astype(np.int32),
                 S.data.astype(np.float64))


def start_block(n, k, seed=10):
    return np.stack([W.rhs_normal(n, seed + r) for r in range(k)])


def wanted(w, k, which):
    return w[::-1][:k] if which == "largest" else w[:k]


def check_pairs(M, r, tol, X0):
    k = r["evals"].shape[0]
    U = r["evecs"]
    assert np.allclose(U @ U.T, np.eye(k), atol=1e-10)
    for i in range(k):
        res = np.linalg.norm(M @ U[i] - r["evals"][i] * U[i])
        assert res <= tol * abs(r["evals"][i]) * (1 + 1e-6) + 1e-13 * np.abs(M).sum(axis=1).max()
        assert abs(res - r["res"][i]) <= 1e-12 * np.abs(M).sum(axis=1).max()
        assert U[i] @ X0[i] >= 0.0


@pytest.mark.parametrize("which", ["largest", "smallest"])
def test_lobpcg_vs_dense_eigh(which):
    A, _, _ = W.varcoef_poisson5(14, seed=3)
    M = dense(A)
    w, V = np.linalg.eigh(M)
    k = 4
    X0 = start_block(A.n_rows, k)
    r = L.lobpcg(A, k, X0, which=which, tol=1e-10, max_iter=5000)
    assert r["state"] == O.CONVERGED and r["iterations"] > 0
    idx = np.arange(A.n_rows - 1, A.n_rows - 1 - k, -1) if which == "largest" else np.arange(k)
    scale = np.abs(w).max()
    assert np.abs(r["evals"] - w[idx]).max() <= 1e-12 * scale
    for i in range(k):
        ref = V[:, idx[i]] * np.sign(V[:, idx[i]] @ X0[i])
        gap = np.min(np.abs(np.delete(w, idx[i]) - w[idx[i]]))
        assert np.linalg.norm(r["evecs"][i] - ref) <= 10 * 1e-10 * abs(w[idx[i]]) / gap + 1e-12
    check_pairs(M, r, 1e-10, X0)


@pytest.mark.parametrize("which", ["largest", "smallest"])
def test_lobpcg_laplacian_closed_form(which):
    nx, ny = 11, 9
    Tx = 2 * np.eye(nx) - np.eye(nx, k=1) - np.eye(nx, k=-1)
    Ty = 2 * np.eye(ny) - np.eye(ny, k=1) - np.eye(ny, k=-1)
    A = csr_of_dense(np.kron(np.eye(ny), Tx) + np.kron(Ty, np.eye(nx)))
    lam = np.sort([4 - 2 * math.cos(p * math.pi / (nx + 1)) - 2 * math.cos(q * math.pi / (ny + 1))
                   for p in range(1, nx + 1) for q in range(1, ny + 1)])
    k = 3
    X0 = start_block(A.n_rows, k, seed=2)
    r = L.lobpcg(A, k, X0, which=which, tol=1e-11, max_iter=5000)
    assert r["state"] == O.CONVERGED
    assert np.abs(r["evals"] - wanted(lam, k, which)).max() <= 1e-12 * 8
    check_pairs(dense(A), r, 1e-11, X0)


def test_lobpcg_invariant_start_block():
    # X0 in the span of e_3, e_17, e_40 of diag(1..50): exact pairs before any iteration
    n = 50
    A = csr_of_dense(np.diag(np.arange(1.0, n + 1.0)))
    X0 = np.zeros((3, n))
    X0[0, [3, 17]] = [1.0, 2.0]
    X0[1, [17, 40]] = [-1.0, 0.5]
    X0[2, [3, 40]] = [0.25, 3.0]
    r = L.lobpcg(A, 3, X0, which="largest", tol=1e-12)
    assert r["state"] == O.CONVERGED and r["iterations"] == 0
    assert np.abs(r["evals"] - [41.0, 18.0, 4.0]).max() <= 1e-13 * 41
    for i, c in enumerate([40, 17, 3]):
        assert abs(abs(r["evecs"][i][c]) - 1.0) <= 1e-13


@pytest.mark.parametrize("which", ["largest", "smallest"])
def test_lobpcg_ritz_values_monotone_and_interlaced(which):
    A, _, _ = W.varcoef_poisson5(12, seed=5)
    w = np.linalg.eigvalsh(dense(A))
    k = 3
    X0 = start_block(A.n_rows, k, seed=4)
    tw = wanted(w, k, which)
    sgn = 1.0 if which == "largest" else -1.0
    prev = None
    for it in range(0, 8):
        r = L.lobpcg(A, k, X0, which=which, tol=1e-300, max_iter=it)
        assert r["state"] == O.MAX_ITER and r["iterations"] == it
        th = r["evals"]
        assert np.all(sgn * (tw - th) >= -1e-12 * np.abs(w).max())          # interlacing
        if prev is not None:
            assert np.all(sgn * (th - prev) >= -1e-12 * np.abs(w).max())    # Courant-Fischer
            assert np.any(sgn * (th - prev) > 1e-8)                         # and a real step
        prev = th


def test_lobpcg_agrees_with_lanczos():
    from oracle.eigsh import eigsh
    A, _, _ = W.varcoef_poisson5(40, seed=1)
    k = 4
    X0 = start_block(A.n_rows, k, seed=7)
    for which in ("largest", "smallest"):
        r = L.lobpcg(A, k, X0, which=which, tol=1e-10, max_iter=20000)
        z = eigsh(A, k, X0[0], which=which, tol=1e-12)
        assert r["state"] == z["state"] == O.CONVERGED
        assert np.abs(r["evals"] - z["evals"]).max() <= 1e-12 * np.abs(dense(A)).sum(axis=1).max()


def knyazev_ritz(M, X0, k, which, iters, tinv=None):
    """Ritz values after `iters` steps of Rayleigh-Ritz on span{X_i, T R_i, X_{i-1}}
    (Knyazev's formulation; LOBPCG's basis [X, W, P] spans the same space), by numpy QR
    and eigh on the dense matrix: independent of the oracle's blocks and factorizations."""
    def rr(Q):
        Q, _ = np.linalg.qr(Q)
        w, V = np.linalg.eigh(Q.T @ M @ Q)
        idx = np.arange(len(w) - 1, len(w) - 1 - k, -1) if which == "largest" else np.arange(k)
        return w[idx], Q @ V[:, idx]
    th, X = rr(X0.T)
    Xprev = None
    for _ in range(iters):
        R = M @ X - X * th
        W = R if tinv is None else R * tinv[:, None]
        blocks = [X, W] + ([Xprev] if Xprev is not None else [])
        Xprev = X
        th, X = rr(np.hstack(blocks))
    return th


@pytest.mark.parametrize("jacobi", [False, True])
@pytest.mark.parametrize("which", ["largest", "smallest"])
def test_lobpcg_trial_space_is_knyazevs(which, jacobi):
    A, _, _ = W.varcoef_poisson5(10, seed=2)
    M = dense(A)
    k = 3
    X0 = start_block(A.n_rows, k, seed=6)
    tinv = 1.0 / np.diag(M) if jacobi else None
    for it in (1, 2, 3):
        r = L.lobpcg(A, k, X0, which=which, tol=1e-300, max_iter=it, jacobi=jacobi)
        ref = knyazev_ritz(M, X0, k, which, it, tinv)
        assert np.abs(r["evals"] - ref).max() <= 1e-10 * np.abs(M).sum(axis=1).max(), (it, r["evals"], ref)


def test_lobpcg_jacobi_vs_dense_eigh():
    A, _, _ = W.varcoef_poisson5(14, seed=3)
    M = dense(A)
    w = np.linalg.eigvalsh(M)
    k = 4
    X0 = start_block(A.n_rows, k)
    r = L.lobpcg(A, k, X0, which="smallest", tol=1e-10, max_iter=5000, jacobi=True)
    p = L.lobpcg(A, k, X0, which="smallest", tol=1e-10, max_iter=5000)
    assert r["state"] == O.CONVERGED and r["iterations"] < p["iterations"] / 2
    assert np.abs(r["evals"] - w[:k]).max() <= 1e-12 * np.abs(w).max()
    check_pairs(M, r, 1e-10, X0)


def test_lobpcg_jacobi_needs_a_positive_diagonal():
    A, _, _ = W.varcoef_poisson5(6, seed=1)
    v = A.vals.copy()
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))
    v[np.flatnonzero(rows == A.col)[3]] = -1.0
    with pytest.raises(ValueError):
        L.lobpcg(A, 2, start_block(A.n_rows, 2), jacobi=True, vals=v)
