"""Pins of the oracle's Lanczos eigensolver (oracle/eigsh.py) and of the
Hellmann-Feynman eigenvalue gradient, against facts fixed by the mathematics.

  eigenpairs  numpy.linalg.eigh of the dense matrix (an independent library routine,
              on A itself rather than on the Lanczos tridiagonal); the closed-form
              spectrum of the 5-point Laplacian on an Nx x Ny grid (Nx != Ny, so the
              extreme eigenvalues are simple); exact termination when v0 lies in an
              invariant subspace (two eigenvector components: two steps, beta = 0),
              and BREAKDOWN when that subspace is smaller than k; the stop test's
              residual bound on the returned pairs, and the Lanczos identity that
              makes beta_m |s[m-1]| their true residual; orthonormal vectors with
              <u, v0> >= 0; MAX_ITER at the dimension cap; thick restart (a
              basis of 12 or 30 vectors) reaching dense eigh's pairs, with the
              Lanczos relation intact.
  gradient    central finite differences of dense eigenvalues under a symmetric
              perturbation of the stored values, under the pages' 1e-5 bar (torch-sla,
              paperpeel page, section 4.3, Table 5); the closed form u_i u_j on a
              diagonal matrix.
The module under test can be replaced through SLA_ORACLE_EIGSH (a path to a modified
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
    path = os.environ.get("SLA_ORACLE_EIGSH")
    if not path:
        from oracle import eigsh as E
        return E
    spec = importlib.util.spec_from_file_location("oracle.eigsh_under_test", path)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    spec.loader.exec_module(mod)
    return mod


E = _load()


def dense(A, vals=None):
    v = A.vals if vals is None else vals
    return sp.csr_matrix((v, A.col, A.row_ptr.astype(np.int64)), shape=(A.n_rows, A.n_cols)).toarray()


def csr_of_dense(M):
    S = sp.csr_matrix(M)
    S.sort_indices()
    return W.CSR(M.shape[0], M.shape[1], S.indptr.astype(np.int32), S.indices.astype(np.int32),
                 S.data.astype(np.float64))


def laplacian_rect(nx, ny):
    """5-point Laplacian (4, -1) on an nx x ny grid, unknown (a, c) -> a nx + c."""
    Tx = 2 * np.eye(nx) - np.eye(nx, k=1) - np.eye(nx, k=-1)
    Ty = 2 * np.eye(ny) - np.eye(ny, k=1) - np.eye(ny, k=-1)
    return csr_of_dense(np.kron(np.eye(ny), Tx) + np.kron(Ty, np.eye(nx)))


def check_pairs(A, r, tol):
    M = dense(A)
    k = r["evals"].shape[0]
    U = r["evecs"]
    assert np.allclose(U @ U.T, np.eye(k), atol=1e-10)
    for i in range(k):
        res = np.linalg.norm(M @ U[i] - r["evals"][i] * U[i])
        assert res <= 2 * tol * abs(r["evals"][i]) + 1e-13
        # the Lanczos identity A V_m s = V_m T_m s + beta_m v_{m+1} (e_m^T s): the true
        # residual of a Ritz pair is beta_m |s[m-1]|, the estimate the stop test uses
        assert abs(res - r["res_est"][i]) <= 1e-12 * abs(r["evals"][i])


@pytest.mark.parametrize("which", ["largest", "smallest"])
def test_eigsh_vs_dense_eigh(which):
    A, _, _ = W.varcoef_poisson5(14, seed=3)
    M = dense(A)
    w, V = np.linalg.eigh(M)
    v0 = W.rhs_normal(A.n_rows, 1)
    k = 4
    r = E.eigsh(A, k, v0, which=which, tol=1e-12)
    assert r["state"] == O.CONVERGED and k <= r["iterations"] <= A.n_rows
    idx = np.arange(A.n_rows - 1, A.n_rows - 1 - k, -1) if which == "largest" else np.arange(k)
    scale = np.abs(w).max()
    assert np.abs(r["evals"] - w[idx]).max() <= 1e-12 * scale
    for i in range(k):
        ref = V[:, idx[i]] * np.sign(V[:, idx[i]] @ v0)
        assert np.linalg.norm(r["evecs"][i] - ref) <= 1e-9
        assert r["evecs"][i] @ v0 >= 0
    check_pairs(A, r, 1e-12)


@pytest.mark.parametrize("which", ["largest", "smallest"])
def test_eigsh_laplacian_closed_form(which):
    nx, ny = 11, 9
    A = laplacian_rect(nx, ny)
    lam = np.sort([4 - 2 * math.cos(p * math.pi / (nx + 1)) - 2 * math.cos(q * math.pi / (ny + 1))
                   for p in range(1, nx + 1) for q in range(1, ny + 1)])
    k = 3
    ref = lam[::-1][:k] if which == "largest" else lam[:k]
    assert np.min(np.abs(np.diff(ref))) > 1e-3     # simple eigenvalues
    r = E.eigsh(A, k, W.rhs_normal(A.n_rows, 2), which=which, tol=1e-11)
    assert r["state"] == O.CONVERGED
    assert np.abs(r["evals"] - ref).max() <= 1e-12
    check_pairs(A, r, 1e-11)


def test_eigsh_invariant_subspace_and_breakdown():
    n = 50
    d = np.arange(1.0, n + 1.0)
    A = csr_of_dense(np.diag(d))
    v0 = np.zeros(n)
    v0[[6, 31]] = [3.0, -2.0]          # eigenvectors e_6 (lambda 7) and e_31 (lambda 32)
    r = E.eigsh(A, 2, v0, which="largest", tol=1e-12)
    assert r["state"] == O.CONVERGED and r["iterations"] == 2
    assert np.abs(r["evals"] - [32.0, 7.0]).max() <= 1e-13
    assert abs(abs(r["evecs"][0][31]) - 1.0) <= 1e-13 and r["evecs"][0][31] < 0   # <u, v0> >= 0
    assert abs(r["evecs"][1][6] - 1.0) <= 1e-13
    r3 = E.eigsh(A, 3, v0, which="largest", tol=1e-12)
    assert r3["state"] == O.BREAKDOWN and r3["iterations"] == 2


def test_eigsh_dimension_cap():
    A, _, _ = W.varcoef_poisson5(20, seed=4)
    r = E.eigsh(A, 3, W.rhs_normal(A.n_rows, 3), which="smallest", tol=1e-14, max_dim=12)
    assert r["state"] == O.MAX_ITER and r["iterations"] == 12
    # Ritz values of a partial Krylov space lie inside the spectrum (interlacing)
    w = np.linalg.eigvalsh(dense(A))
    assert np.all(r["evals"] >= w[0] - 1e-12) and np.all(r["evals"] <= w[-1] + 1e-12)
    assert np.all(r["evals"][:3] >= w[:3] - 1e-12)


@pytest.mark.parametrize("which,m", [("smallest", 30), ("largest", 12)])
def test_eigsh_thick_restart(which, m):
    # a basis of m vectors restarted from the kept Ritz vectors: the same eigenpairs as
    # dense eigh, and the Lanczos relation (true residual = beta |s[m-1]|) still holds
    A, _, _ = W.varcoef_poisson5(20, seed=6)
    M = dense(A)
    w, V = np.linalg.eigh(M)
    v0 = W.rhs_normal(A.n_rows, 9)
    k = 4
    r = E.eigsh(A, k, v0, which=which, tol=1e-11, max_dim=m, max_iter=20000)
    assert r["state"] == O.CONVERGED and r["restarts"] > 0
    idx = np.arange(A.n_rows - 1, A.n_rows - 1 - k, -1) if which == "largest" else np.arange(k)
    assert np.abs(r["evals"] - w[idx]).max() <= 1e-12 * np.abs(w).max()
    for i in range(k):
        ref = V[:, idx[i]] * np.sign(V[:, idx[i]] @ v0)
        assert np.linalg.norm(r["evecs"][i] - ref) <= 1e-8
    check_pairs(A, r, 1e-11)
    # without the budget to restart, the same basis size stops at MAX_ITER
    r0 = E.eigsh(A, k, v0, which=which, tol=1e-11, max_dim=m)
    assert r0["state"] == O.MAX_ITER and r0["iterations"] == m


@pytest.mark.parametrize("which", ["largest", "smallest"])
def test_hellmann_feynman_vs_finite_differences(which):
    A, _, _ = W.varcoef_poisson5(10, seed=5)
    k = 3
    r = E.eigsh(A, k, W.rhs_normal(A.n_rows, 4), which=which, tol=1e-13)
    g = np.array([1.0, -0.5, 2.0])
    grad = E.eigsh_grad(A, r["evecs"], g)
    # symmetric perturbation of the stored values (keeps A symmetric)
    rng = np.random.default_rng(8)
    Md = dense(A, rng.standard_normal(A.nnz))
    Md = 0.5 * (Md + Md.T)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))
    dv = Md[rows, A.col]
    h = 1e-5

    def wanted(vals):
        w = np.linalg.eigvalsh(dense(A, vals))
        return w[::-1][:k] if which == "largest" else w[:k]

    fd = (wanted(A.vals + h * dv) - wanted(A.vals - h * dv)) / (2 * h)
    an = float(grad @ dv)
    assert abs(float(g @ fd) - an) <= 1e-7 * abs(an)


def test_hellmann_feynman_closed_form_on_a_diagonal():
    # diag(d) with an off-diagonal pair stored as explicit zeros: u = e_i, so the
    # gradient is g at the entry (i, i) and 0 everywhere else, zeros included
    n = 6
    M = np.diag([1.0, 2.0, 3.0, 5.0, 8.0, 13.0])
    S = sp.csr_matrix(M + 1e-300 * (np.eye(n, k=1) + np.eye(n, k=-1)))
    S.sort_indices()
    A = W.CSR(n, n, S.indptr.astype(np.int32), S.indices.astype(np.int32), np.where(S.data < 1e-200, 0.0, S.data))
    r = E.eigsh(A, 2, np.ones(n), which="largest", tol=1e-13)
    grad = E.eigsh_grad(A, r["evecs"], np.array([1.5, -2.0]))
    rows = np.repeat(np.arange(n), np.diff(A.row_ptr.astype(np.int64)))
    expect = np.where((rows == A.col) & (rows == 5), 1.5, np.where((rows == A.col) & (rows == 4), -2.0, 0.0))
    assert np.abs(grad - expect).max() <= 1e-13
