"""Pins of the oracle's BiCGStab and its nonsymmetric adjoint, against facts fixed by
the mathematics rather than by the oracle.

BiCGStab (van der Vorst, 1992) is the pages' second iterative method (torch-sla,
paperpeel page, section 1 and section 3.1 "Five backends and auto-dispatch").  The
checks below are chosen so that a plausible mistake in orc_bicgstab fails one of them
(tests/test_oracle_mutations.py plants such mistakes):

  solve      dense LU on nonsymmetric convection-diffusion grids within the bound
             that the stop test and the condition number give; a manufactured
             solution; finite termination (with m distinct eigenvalues the residual
             vanishes after at most m iterations in exact arithmetic: r_k =
             Q_k(A) P_k(A) r_0 with P_k the Bi-CG residual polynomial); a multiple of the
             identity and an eigenvector right-hand side (one iteration, stopped
             half-way); SPD systems, where the solution is CG's.
  states     a zero right-hand side, the budget, fixed mode, a breakdown
             <r0, A p> = 0 (a rotation), NaN values.
  adjoint    dense LU for lambda = A^-T g and -lambda_i x_j on a nonsymmetric
             matrix; the homogeneity invariants; central finite differences.
"""
import math

import numpy as np
import pytest
import scipy.sparse as sp

import oracle as O
import workloads as W

EPS = np.finfo(np.float64).eps


def rel_err(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(b))


def dense(A, vals=None):
    v = A.vals if vals is None else vals
    return sp.csr_matrix((v, A.col, A.row_ptr.astype(np.int64)), shape=(A.n_rows, A.n_cols)).toarray()


def csr_of_dense(M):
    S = sp.csr_matrix(M)
    S.sort_indices()
    return W.CSR(M.shape[0], M.shape[1], S.indptr.astype(np.int32), S.indices.astype(np.int32),
                 S.data.astype(np.float64))


# ------------------------------------------------------------------------------- solve
@pytest.mark.parametrize("N,wind", [(8, 100.0), (12, 30.0), (16, 300.0)])
def test_bicgstab_vs_dense_lu(N, wind):
    A = W.convdiff5(N, wind=wind)
    M = dense(A)
    assert np.abs(M - M.T).max() > 0.1          # genuinely nonsymmetric
    b = W.rhs_normal(N * N, 3)
    rtol = 1e-12
    f = O.bicgstab(A, b, rtol=rtol)
    assert f["state"] == O.CONVERGED
    x_lu = np.linalg.solve(M, b)
    # |x - x*| <= |A^-1| |r| <= |A^-1| rtol |b| (plus the drift of the recurrence residual)
    bound = np.linalg.norm(np.linalg.inv(M), 2) * (rtol * np.linalg.norm(b)) * 10 + 1e3 * EPS * np.linalg.norm(x_lu)
    assert np.linalg.norm(f["x"] - x_lu) <= bound
    assert f["res_norm"] <= rtol * f["rhs_norm"]
    assert f["rhs_norm"] == pytest.approx(np.linalg.norm(b), rel=1e-15)


def test_bicgstab_manufactured_solution():
    A = W.convdiff5(20, wind=50.0, shift=0.25)
    xs = np.random.default_rng(4).uniform(-1.0, 1.0, A.n_rows)
    b = dense(A) @ xs
    f = O.bicgstab(A, b, rtol=1e-13)
    assert f["state"] == O.CONVERGED
    assert rel_err(f["x"], xs) <= 1e-11


@pytest.mark.parametrize("n,m", [(30, 2), (30, 3), (50, 4)])
def test_bicgstab_terminates_after_m_eigenvalues(n, m):
    # A = S D S^-1 with m distinct eigenvalues (one negative: indefinite, and S makes
    # A nonsymmetric): its minimal polynomial has degree m, so in exact arithmetic the
    # Bi-CG residual polynomial kills r0 at step m and so does BiCGStab's.
    rng = np.random.default_rng(n + m)
    S = np.eye(n) + 0.3 * rng.standard_normal((n, n)) / math.sqrt(n)
    d = np.resize(np.array([1.0, 2.5, -1.5, 4.0])[:m], n)
    M = S @ np.diag(d) @ np.linalg.inv(S)
    A = csr_of_dense(M)
    b = rng.standard_normal(n)
    f = O.bicgstab(A, b, rtol=1e-12)
    assert f["state"] == O.CONVERGED
    assert f["iterations"] <= m
    assert rel_err(f["x"], np.linalg.solve(M, b)) <= 1e-11


def test_bicgstab_multiple_of_identity():
    n = 37
    A = csr_of_dense(np.eye(n) * 4.0)
    b = np.random.default_rng(5).standard_normal(n)
    f = O.bicgstab(A, b, rtol=1e-14, history=True)
    # v = 4 b, alpha = 1/4 exactly, s = b - b / 4 * 4 = 0: stopped half-way after one
    # iteration with x = b / 4 (every step exact in binary)
    assert f["state"] == O.CONVERGED and f["iterations"] == 1
    assert np.array_equal(f["x"], b / 4.0)
    assert f["history"][1] == 0.0 and f["res_norm"] == 0.0


@pytest.mark.parametrize("N,p,q", [(16, 2, 3), (31, 5, 1)])
def test_bicgstab_eigenvector_one_iteration(N, p, q):
    A = W.poisson5(N)
    i = np.arange(1, N + 1)
    v = np.outer(np.sin(p * np.pi * i / (N + 1)), np.sin(q * np.pi * i / (N + 1))).reshape(-1)
    lam = 4.0 - 2.0 * math.cos(p * math.pi / (N + 1)) - 2.0 * math.cos(q * math.pi / (N + 1))
    f = O.bicgstab(A, v, rtol=1e-10)
    assert f["state"] == O.CONVERGED and f["iterations"] == 1
    assert rel_err(f["x"], v / lam) <= 50 * EPS


def test_bicgstab_on_spd_gives_cgs_solution():
    A, b, _ = W.varcoef_poisson5(14, seed=2)
    M = dense(A)
    x_lu = np.linalg.solve(M, b)
    f = O.bicgstab(A, b, rtol=1e-13)
    g = O.cg(A, b, rtol=1e-13)
    assert f["state"] == O.CONVERGED
    assert rel_err(f["x"], x_lu) <= 1e-10 and rel_err(g["x"], x_lu) <= 1e-10


def test_convdiff_generator():
    # wind 0 gives the Poisson matrix bit for bit; the wind adds only upwind terms
    P, Z = W.poisson5(9), W.convdiff5(9, wind=0.0)
    assert np.array_equal(P.col, Z.col) and np.array_equal(P.vals, Z.vals)
    A = W.convdiff5(9, wind=80.0)
    M = dense(A)
    off = M - np.diag(np.diag(M))
    assert (off <= 0).all() and (np.diag(M) > 0).all()
    # row sums: h (|wx| + |wy|) - h (upwind terms) >= 0 with equality away from walls
    assert (M.sum(1) >= -1e-12).all()
    # batch of winds: same pattern, one row of values per wind
    B = W.convdiff5(9, wind=[0.0, 80.0])
    assert B.vals.shape == (2, A.nnz) and np.array_equal(B.vals[1], A.vals)


# ------------------------------------------------------------------------------ states
def test_bicgstab_zero_rhs_budget_and_fixed():
    A = W.convdiff5(10, wind=60.0)
    n = A.n_rows
    f = O.bicgstab(A, np.zeros(n), rtol=1e-8)
    assert f["state"] == O.CONVERGED and f["iterations"] == 0 and not f["x"].any()
    b = W.rhs_normal(n, 7)
    f = O.bicgstab(A, b, rtol=1e-14, max_iter=3)
    assert f["state"] == O.MAX_ITER and f["iterations"] == 3
    f0 = O.bicgstab(A, b, rtol=1e-8, max_iter=0)
    assert f0["state"] == O.MAX_ITER and f0["iterations"] == 0 and not f0["x"].any()
    K = 7
    h = O.bicgstab(A, b, rtol=0.0, max_iter=K, fixed=True, history=True)
    assert h["state"] == O.MAX_ITER and h["iterations"] == K and h["history"].shape == (K + 1,)
    # the recorded residuals are those of the iterates: |b - A x_K| matches |r_K|
    assert abs(np.linalg.norm(b - dense(A) @ h["x"]) - h["history"][K]) <= 1e-10 * np.linalg.norm(b)


def test_bicgstab_breakdown_on_a_rotation():
    # A = rotation by 90 degrees: <b, A b> = 0 for every b, so <r0, A p0> = 0
    A = csr_of_dense(np.array([[0.0, -1.0], [1.0, 0.0]]))
    f = O.bicgstab(A, np.array([1.0, 2.0]), rtol=1e-10)
    assert f["state"] == O.BREAKDOWN and f["iterations"] == 0 and not f["x"].any()


def test_bicgstab_nan():
    A = W.convdiff5(6, wind=10.0)
    v = A.vals.copy()
    v[5] = np.nan
    f = O.bicgstab(A, W.rhs_normal(A.n_rows, 1), rtol=1e-10, vals=v)
    assert f["state"] == O.NAN and f["iterations"] == 0


# ----------------------------------------------------------------------------- adjoint
@pytest.mark.parametrize("N,wind", [(6, 100.0), (10, 40.0)])
def test_bicgstab_adjoint_vs_dense_lu(N, wind):
    A = W.convdiff5(N, wind=wind)
    M = dense(A)
    b = W.rhs_normal(N * N, 2)
    x = np.linalg.solve(M, b)
    g = np.random.default_rng(9).standard_normal(N * N)
    bw = O.solve_backward(A, x, g, symmetric=False, rtol=1e-13, method="bicgstab")
    assert bw["state"] == O.CONVERGED
    lam = np.linalg.solve(M.T, g)
    assert rel_err(bw["lam"], lam) <= 1e-9
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))
    assert rel_err(bw["gvals"], -lam[rows] * x[A.col]) <= 1e-9
    # without the transpose (symmetric=True on a nonsymmetric A) the answer is wrong
    wrong = O.solve_backward(A, x, g, symmetric=True, rtol=1e-13, method="bicgstab")
    assert rel_err(wrong["lam"], lam) > 1e-3


def test_bicgstab_adjoint_homogeneity_invariants():
    # x(cA, cb) = x(A, b): <dL/dvals, vals> + <dL/db, b> = 0; for L = |x|^2 / 2 the
    # second term is 2 L
    A = W.convdiff5(12, wind=70.0)
    b = W.rhs_normal(A.n_rows, 5)
    f = O.bicgstab(A, b, rtol=1e-14)
    x = f["x"]
    bw = O.solve_backward(A, x, x, symmetric=False, rtol=1e-14, method="bicgstab")
    L2 = float(x @ x)
    assert float(bw["lam"] @ b) == pytest.approx(L2, rel=1e-10)
    assert float(bw["gvals"] @ A.vals) == pytest.approx(-L2, rel=1e-10)


def test_bicgstab_adjoint_directional_fd():
    A = W.convdiff5(10, wind=50.0)
    b = W.rhs_normal(A.n_rows, 6)
    rng = np.random.default_rng(12)
    dv, db = rng.standard_normal(A.nnz), rng.standard_normal(A.n_rows)

    def loss(vals, bb):
        x = O.bicgstab(A, bb, rtol=1e-14, vals=vals)["x"]
        return 0.5 * float(x @ x)

    x = O.bicgstab(A, b, rtol=1e-14)["x"]
    bw = O.solve_backward(A, x, x, symmetric=False, rtol=1e-14, method="bicgstab")
    h = 1e-6
    fd = (loss(A.vals + h * dv, b + h * db) - loss(A.vals - h * dv, b - h * db)) / (2 * h)
    an = float(bw["gvals"] @ dv + bw["lam"] @ db)
    assert abs(fd - an) <= 1e-6 * abs(an)
