"""Pins of the CPU oracle against facts fixed by the mathematics, not by the oracle.

Each check is chosen so that a plausible mistake in the oracle fails it:
a dropped term, a wrong sign, a wrong or transposed index.

  SpMV       exact integer arithmetic; closed-form eigenpairs of the 5-point
             Laplacian; scipy.sparse products (an independent library routine).
  CG         dense LU on small grids within the condition-number bound; a
             manufactured solution; one iteration on an eigenvector; m
             iterations on m modes; exact rationals on a 2 x 2 grid
             (tests/golden/poisson2x2.json); the stopping and breakdown cases.
  adjoint    dense LU for lambda = A^-T g and -lambda_i x_j; closed forms on an
             eigenvector right-hand side; the homogeneity invariants; central
             finite differences under the pages' 1e-5 bar (torch-sla, paperpeel
             section 4.3 "Gradient Verification"); reverse-mode differentiation
             through the converged CG iterations themselves (section 4.2).
  transpose  involution, symmetric fixed point, scipy's transpose.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.sparse as sp

import oracle as O
import workloads as W

EPS = np.finfo(np.float64).eps
HERE = os.path.dirname(os.path.abspath(__file__))


def rel_err(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(b))


def dense(A, vals=None):
    v = A.vals if vals is None else vals
    return sp.csr_matrix((v, A.col, A.row_ptr.astype(np.int64)), shape=(A.n_rows, A.n_cols)).toarray()


def sin_mode(N, p, q):
    i = np.arange(1, N + 1)
    v = np.outer(np.sin(p * np.pi * i / (N + 1)), np.sin(q * np.pi * i / (N + 1))).reshape(-1)
    lam = 4.0 - 2.0 * math.cos(p * math.pi / (N + 1)) - 2.0 * math.cos(q * math.pi / (N + 1))
    return v, lam


def cond_poisson(N):
    # extreme eigenvalues 4 - 4cos(pi/(N+1)) and 4 + 4cos(pi/(N+1))
    c = math.cos(math.pi / (N + 1))
    return (1 + c) / (1 - c)


# ----------------------------------------------------------------------------- SpMV
def test_spmv_integer_exact():
    rng = np.random.default_rng(11)
    A = W.poisson5(17)
    xi = rng.integers(-2 ** 20, 2 ** 20, A.n_cols)
    # brute force in integers: every product and partial sum is exact
    y_int = np.zeros(A.n_rows, np.int64)
    for i in range(A.n_rows):
        for k in range(A.row_ptr[i], A.row_ptr[i + 1]):
            y_int[i] += int(A.vals[k]) * int(xi[A.col[k]])
    y = O.spmv(A, xi.astype(np.float64))
    assert np.array_equal(y, y_int.astype(np.float64))


@pytest.mark.parametrize("N,p,q", [(64, 3, 5), (31, 1, 1), (20, 20, 7)])
def test_spmv_sin_eigenpairs(N, p, q):
    A = W.poisson5(N)
    v, lam = sin_mode(N, p, q)
    r = O.spmv(A, v) - lam * v
    assert np.linalg.norm(r) <= 8 * 5 * EPS * 8.0 * np.linalg.norm(v)
    # a wrong neighbour index breaks the eigen-relation by O(1)
    assert np.linalg.norm(r) < 1e-12 * np.linalg.norm(lam * v)


def test_spmv_matches_scipy_on_fem_and_varcoef():
    rng = np.random.default_rng(3)
    A, _ = W.fem_p1_batched(nv=24, B=2, seed=5)
    x = rng.standard_normal(A.n_cols)
    M = sp.csr_matrix((A.vals[1], A.col, A.row_ptr), shape=(A.n_rows, A.n_cols))
    ref = M @ x
    y = O.spmv(A, x, vals=A.vals[1])
    scale = abs(M) @ abs(x)
    assert np.all(np.abs(y - ref) <= 16 * EPS * scale)
    V, _, _ = W.varcoef_poisson5(20, seed=2)
    x = rng.standard_normal(V.n_cols)
    M = sp.csr_matrix((V.vals, V.col, V.row_ptr), shape=(V.n_rows, V.n_cols))
    assert np.all(np.abs(O.spmv(V, x) - M @ x) <= 16 * EPS * (abs(M) @ abs(x)))


def test_spmv_transposed_matches_dense_on_nonsymmetric():
    rng = np.random.default_rng(4)
    A = W.poisson5(9)
    vals = rng.standard_normal(A.nnz)            # same pattern, non-symmetric values
    x = rng.standard_normal(A.n_rows)
    D = dense(A, vals)
    assert np.allclose(O.spmv_transposed(A, x, vals=vals), D.T @ x, rtol=0, atol=1e-13)
    assert np.allclose(O.spmv(A, x, vals=vals), D @ x, rtol=0, atol=1e-13)
    assert not np.allclose(D, D.T)


def exact_dot(a, b):
    """sum a_i b_i in exact rational arithmetic, rounded once (float(Fraction) rounds
    correctly)."""
    from fractions import Fraction
    return float(sum((Fraction(x) * Fraction(y) for x, y in zip(a.tolist(), b.tolist())), Fraction(0)))


def test_dot_is_the_exact_sum_rounded():
    # the inner product is the exact sum rounded once, not one summation order's result
    a = np.array([1e16, 1.0, -1e16, 1.0])
    b = np.ones(4)
    assert O.dot(a, b) == 2.0            # sequential fp64 gives 1.0, pairwise 0.0
    a = np.array([1.0 + 2.0 ** -30, 1.0])
    b = np.array([1.0 - 2.0 ** -30, -1.0])
    assert O.dot(a, b) == -(2.0 ** -60)  # needs the product's rounding error
    rng = np.random.default_rng(0)
    for trial in range(20):
        n = int(rng.integers(1, 2000))
        a = rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 6, n)
        b = rng.standard_normal(n)
        if trial % 2:                    # heavy cancellation: append the negated products
            a, b = np.concatenate([a, -a * (1 + 2.0 ** -40)]), np.concatenate([b, b])
        e = exact_dot(a, b)
        assert abs(O.dot(a, b) - e) <= np.spacing(abs(e)), trial


# ----------------------------------------------------------------------------- Jacobi PCG
def scaled(A, s):
    """S A S for S = diag(s): entry (i, j) times s_i s_j."""
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))
    return W.CSR(A.n_rows, A.n_cols, A.row_ptr, A.col, A.vals * s[rows] * s[A.col])


def test_pcg_is_cg_bit_for_bit_on_a_constant_diagonal():
    # diagonal 4: z = r / 4 and every scaling by a power of two is exact, so PCG and CG
    # produce the same iterates to the last bit
    A = W.poisson5(20)
    b = W.rhs_uniform(A.n_rows, 3)
    f = O.cg(A, b, rtol=1e-10, history=True)
    g = O.cg(A, b, rtol=1e-10, history=True, jacobi=True)
    assert g["iterations"] == f["iterations"] and g["state"] == f["state"]
    assert np.array_equal(g["x"], f["x"]) and np.array_equal(g["history"], f["history"])


def test_pcg_on_a_diagonal_matrix_takes_one_iteration():
    n = 300
    d = np.random.default_rng(4).uniform(0.1, 10.0, n)
    A = W.CSR(n, n, np.arange(n + 1, dtype=np.int64), np.arange(n, dtype=np.int32), d)
    b = W.rhs_normal(n, 5)
    g = O.cg(A, b, rtol=1e-12, jacobi=True)
    assert g["iterations"] == 1 and g["state"] == O.CONVERGED
    assert np.allclose(g["x"], b / d, rtol=1e-15, atol=0)
    f = O.cg(A, b, rtol=1e-12)                 # plain CG needs many more
    assert f["iterations"] > 20


@pytest.mark.parametrize("N", [12, 20])
def test_pcg_on_a_rescaled_matrix_follows_cg(N):
    # PCG with M = diag(S A S) on S A S x' = S b is CG on A / 4 (A = 5-point Poisson,
    # diagonal 4): the same Krylov iterates, x' = S^-1 x, iteration for iteration
    A = W.poisson5(N)
    s = np.random.default_rng(N).uniform(0.3, 3.0, A.n_rows)
    b = W.rhs_normal(A.n_rows, 6)
    f = O.cg(A, b, rtol=1e-10, history=True)
    g = O.cg(scaled(A, s), s * b, rtol=0.0, max_iter=f["iterations"], fixed=True, jacobi=True)
    assert rel_err(g["x"] * s, f["x"]) <= 1e-8
    # the preconditioned residual norms <r', M^-1 r'> = <r, r> / 4 track CG's
    h = O.cg(scaled(A, s), s * b, rtol=1e-10, jacobi=True)
    assert abs(h["iterations"] - f["iterations"]) <= 2
    # plain CG on the rescaled matrix is far slower
    assert O.cg(scaled(A, s), s * b, rtol=1e-10)["iterations"] > 1.5 * f["iterations"]


def test_pcg_vs_dense_lu_varcoef():
    A, b, _ = W.varcoef_poisson5(14, seed=2)
    D = dense(A)
    xs = np.linalg.solve(D, b)
    g = O.cg(A, b, rtol=1e-12, jacobi=True)
    assert g["state"] == O.CONVERGED
    assert rel_err(g["x"], xs) <= np.linalg.cond(D) * 1e-12
    f = O.cg(A, b, rtol=1e-12)
    assert g["iterations"] < f["iterations"]   # the coefficient jumps make Jacobi pay


def test_pcg_invalid_diagonal_and_adjoint():
    A = W.poisson5(10)
    b = W.rhs_uniform(A.n_rows, 1)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))
    v = A.vals.copy()
    v[np.nonzero(rows == A.col)[0][7]] = 0.0
    g = O.cg(A, b, vals=v, jacobi=True)
    assert g["state"] == O.NOT_SPD and g["iterations"] == 0 and not np.any(g["x"])
    v[np.nonzero(rows == A.col)[0][7]] = np.nan
    assert O.cg(A, b, vals=v, jacobi=True)["state"] == O.NAN
    assert O.cg(A, np.zeros(A.n_rows), vals=v, jacobi=True)["state"] == O.CONVERGED   # b = 0 first
    # the adjoint with Jacobi solves the same system: lambda = A^-1 g
    A2, b2, _ = W.varcoef_poisson5(10, seed=4)
    x = O.cg(A2, b2, rtol=1e-12, jacobi=True)["x"]
    bw = O.solve_backward(A2, x, x, symmetric=True, rtol=1e-12, jacobi=True)
    lam = np.linalg.solve(dense(A2), x)
    assert rel_err(bw["lam"], lam) <= 1e-9
    rows2 = np.repeat(np.arange(A2.n_rows), np.diff(A2.row_ptr.astype(np.int64)))
    assert np.array_equal(bw["gvals"], -(bw["lam"][rows2] * x[A2.col]))


# ----------------------------------------------------------------------------- CG
@pytest.mark.parametrize("N", [4, 8, 16])
def test_cg_vs_dense_lu(N):
    A = W.poisson5(N)
    b = W.rhs_uniform(N * N, 0)
    rtol = 1e-10
    r = O.cg(A, b, rtol=rtol)
    assert r["state"] == O.CONVERGED
    x_lu = np.linalg.solve(dense(A), b)
    err = np.linalg.norm(r["x"] - x_lu) / np.linalg.norm(x_lu)
    assert err <= cond_poisson(N) * rtol
    # the reported residual is the recurrence residual; the true one agrees closely
    true_res = np.linalg.norm(b - dense(A) @ r["x"])
    assert r["res_norm"] <= rtol * r["rhs_norm"]
    assert abs(true_res - r["res_norm"]) <= 1e-3 * rtol * r["rhs_norm"] + 1e3 * EPS * r["rhs_norm"]


def test_cg_manufactured_solution_fem():
    A, _ = W.fem_p1_batched(nv=12, B=1, seed=1)
    rng = np.random.default_rng(8)
    xs = rng.standard_normal(A.n_rows)
    D = dense(A, A.vals[0])
    b = D @ xs
    r = O.cg(A, b, rtol=1e-12, vals=A.vals[0])
    assert r["state"] == O.CONVERGED
    kappa = np.linalg.cond(D)
    assert np.linalg.norm(r["x"] - xs) / np.linalg.norm(xs) <= kappa * 1e-12


@pytest.mark.parametrize("N,p,q", [(64, 3, 5), (16, 2, 9)])
def test_cg_eigenvector_one_iteration(N, p, q):
    A = W.poisson5(N)
    v, lam = sin_mode(N, p, q)
    r = O.cg(A, v, rtol=1e-10)
    assert r["iterations"] == 1 and r["state"] == O.CONVERGED
    assert np.linalg.norm(r["x"] - v / lam) <= 1e-13 * np.linalg.norm(v / lam)


def test_cg_m_modes_m_iterations():
    N = 32
    A = W.poisson5(N)
    modes = [(1, 1), (2, 5), (7, 3)]          # three distinct eigenvalues
    lams = [sin_mode(N, p, q)[1] for p, q in modes]
    assert len(set(np.round(lams, 12))) == 3
    b = sum(sin_mode(N, p, q)[0] * (i + 1) for i, (p, q) in enumerate(modes))
    r = O.cg(A, b, rtol=1e-10)
    assert r["iterations"] == 3
    x_exact = sum(sin_mode(N, p, q)[0] * (i + 1) / lam for i, ((p, q), lam) in
                  enumerate(zip(modes, lams)))
    assert np.linalg.norm(r["x"] - x_exact) <= 1e-12 * np.linalg.norm(x_exact)


def _golden2x2():
    with open(os.path.join(HERE, "golden", "poisson2x2.json")) as f:
        g = json.load(f)
    A = W.CSR(4, 4, np.array(g["row_ptr"], np.int32), np.array(g["col"], np.int32),
              np.array(g["vals"], np.float64))
    fr = lambda xs: np.array([float(Fraction(s)) for s in xs])
    return g, A, np.array(g["b"], np.float64), fr(g["x"]), fr(g["lambda"])


def test_golden_2x2_matches_generator_and_exact_solution():
    g, A, b, x, lam = _golden2x2()
    P = W.poisson5(2)
    assert np.array_equal(P.row_ptr, A.row_ptr) and np.array_equal(P.col, A.col)
    assert np.array_equal(P.vals, A.vals)
    r = O.cg(A, b, rtol=1e-14)
    assert r["iterations"] == g["cg_iterations_exact_arithmetic"]
    assert np.allclose(r["x"], x, rtol=0, atol=4 * EPS)
    bw = O.solve_backward(A, r["x"], r["x"], symmetric=True, rtol=1e-14)
    assert np.allclose(bw["lam"], lam, rtol=0, atol=4 * EPS)
    rows = np.repeat(np.arange(4), np.diff(A.row_ptr))
    assert np.allclose(bw["gvals"], -lam[rows] * x[A.col], rtol=0, atol=4 * EPS)


def test_cg_zero_rhs_and_stopping_cases():
    A = W.poisson5(8)
    r = O.cg(A, np.zeros(64), rtol=1e-10)
    assert r["iterations"] == 0 and r["state"] == O.CONVERGED and not np.any(r["x"])
    b = W.rhs_uniform(64, 1)
    r = O.cg(A, b, rtol=1e-10, max_iter=1)
    assert r["iterations"] == 1 and r["state"] == O.MAX_ITER
    D = dense(A)
    alpha0 = (b @ b) / (b @ D @ b)           # one steepest-descent step from 0
    assert np.allclose(r["x"], alpha0 * b, rtol=1e-14, atol=0)
    r = O.cg(A, b, rtol=0.0, max_iter=37, fixed=True)
    assert r["iterations"] == 37 and r["state"] == O.MAX_ITER
    r2 = O.cg(A, b, rtol=1e-3, atol=1e-1)   # atol dominates when larger
    assert r2["res_norm"] <= 1e-1 and r2["state"] == O.CONVERGED


def test_cg_breakdowns():
    A = W.poisson5(6)
    b = W.rhs_uniform(36, 2)
    neg = W.CSR(A.n_rows, A.n_cols, A.row_ptr, A.col, -A.vals)
    r = O.cg(neg, b)
    assert r["state"] == O.NOT_SPD and r["iterations"] == 0 and not np.any(r["x"])
    bad = A.vals.copy()
    bad[7] = np.nan
    r = O.cg(A, b, vals=bad)
    assert r["state"] == O.NAN and r["iterations"] == 0
    # indefinite: shift the spectrum of the 6x6 Laplacian so that some eigenvalues are negative
    sh = A.vals.copy()
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr))
    sh[rows == A.col] -= 4.0
    r = O.cg(A, b, vals=sh, max_iter=1000)
    assert r["state"] == O.NOT_SPD


# ----------------------------------------------------------------------------- adjoint
@pytest.mark.parametrize("N", [5, 12])
def test_adjoint_vs_dense_lu(N):
    A = W.poisson5(N)
    b = W.rhs_uniform(N * N, 0)
    r = O.cg(A, b, rtol=1e-13)
    g = np.random.default_rng(1).standard_normal(N * N)
    bw = O.solve_backward(A, r["x"], g, symmetric=True, rtol=1e-13)
    D = dense(A)
    lam = np.linalg.solve(D.T, g)
    assert np.linalg.norm(bw["lam"] - lam) <= 1e-11 * np.linalg.norm(lam)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr))
    ref = -lam[rows] * np.linalg.solve(D, b)[A.col]
    assert np.linalg.norm(bw["gvals"] - ref) <= 1e-11 * np.linalg.norm(ref)
    # transposed orientation would give -lam_j x_i: must be far from the answer
    wrong = -lam[A.col] * np.linalg.solve(D, b)[rows]
    assert np.linalg.norm(wrong - ref) > 1e-3 * np.linalg.norm(ref)


def test_adjoint_transpose_path_equals_symmetric_path():
    A = W.varcoef_poisson5(12, seed=3)[0]
    b = W.rhs_uniform(A.n_rows, 4)
    r = O.cg(A, b, rtol=1e-12)
    g = r["x"].copy()
    s = O.solve_backward(A, r["x"], g, symmetric=True, rtol=1e-12)
    t = O.solve_backward(A, r["x"], g, symmetric=False, rtol=1e-12)
    # A is exactly symmetric, so its canonical transpose is A itself, bit for bit
    assert np.array_equal(s["lam"], t["lam"]) and np.array_equal(s["gvals"], t["gvals"])
    assert s["iterations"] == t["iterations"]


def test_adjoint_nonsymmetric_runs_on_the_transpose():
    # With a non-symmetric A (symmetric=False) the adjoint CG must run on A^T.
    # One CG step is the same for A and A^T (g'Ag = g'A'g); the second is not.
    # Expected values: two CG steps written out on numpy's dense transpose.
    rng = np.random.default_rng(21)
    A = W.poisson5(6)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr))
    vals = A.vals + 0.3 * (rows < A.col) * rng.uniform(0.5, 1.0, A.nnz)   # upper part only
    D = dense(A, vals)
    assert not np.allclose(D, D.T)
    g = rng.standard_normal(A.n_rows)
    x = rng.standard_normal(A.n_rows)
    T = D.T
    a0 = (g @ g) / (g @ T @ g)
    r1 = g - a0 * (T @ g)
    p1 = r1 + ((r1 @ r1) / (g @ g)) * g
    lam2 = a0 * g + ((r1 @ r1) / (p1 @ T @ p1)) * p1
    bw = O.solve_backward(A, x, g, symmetric=False, rtol=0.0, max_iter=2, fixed=True, vals=vals)
    assert bw["iterations"] == 2
    assert np.linalg.norm(bw["lam"] - lam2) <= 1e-13 * np.linalg.norm(lam2)
    assert np.array_equal(bw["gvals"], -(bw["lam"][rows] * x[A.col]))


@pytest.mark.parametrize("N,p,q", [(64, 3, 5), (10, 4, 4)])
def test_adjoint_eigenvector_closed_form(N, p, q):
    A = W.poisson5(N)
    v, lam = sin_mode(N, p, q)
    r = O.cg(A, v, rtol=1e-12)
    bw = O.solve_backward(A, r["x"], r["x"], symmetric=True, rtol=1e-12)   # L = 0.5|x|^2
    assert bw["iterations"] == 1
    assert np.linalg.norm(bw["lam"] - v / lam ** 2) <= 1e-13 * np.linalg.norm(v / lam ** 2)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr))
    ref = -v[rows] * v[A.col] / lam ** 3
    assert np.max(np.abs(bw["gvals"] - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_adjoint_homogeneity_invariants():
    # x(cA, cb) = x(A, b)  =>  <dL/dvals, vals> + <dL/db, b> = 0 for any L(x);
    # for L = 0.5|x|^2 also <dL/db, b> = 2L and <dL/dvals, vals> = -2L.
    A, bb = W.fem_p1_batched(nv=20, B=1, seed=7)
    vals, b = A.vals[0], bb[0]
    r = O.cg(A, b, rtol=1e-13, vals=vals)
    L = 0.5 * float(r["x"] @ r["x"])
    bw = O.solve_backward(A, r["x"], r["x"], symmetric=True, rtol=1e-13, vals=vals)
    gb_b = float(bw["lam"] @ b)
    gv_v = float(bw["gvals"] @ vals)
    assert abs(gb_b - 2 * L) <= 1e-9 * 2 * L
    assert abs(gv_v + 2 * L) <= 1e-9 * 2 * L
    assert abs(gb_b + gv_v) <= 1e-9 * 2 * L


@pytest.mark.parametrize("N", [16, 64])
def test_adjoint_directional_fd(N):
    # central differences of L(x) = sum (x - t)^2 along symmetric random directions,
    # CG at tight tolerance for every evaluation; bar 1e-5 relative (pages' figure)
    A = W.varcoef_poisson5(N, seed=1)[0]
    rng = np.random.default_rng(5)
    b = rng.uniform(0, 1, A.n_rows)
    t = rng.uniform(0, 1, A.n_rows)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr))
    # symmetric perturbation of the stored values keeps A SPD for small h
    key = np.minimum(rows, A.col).astype(np.int64) * A.n_rows + np.maximum(rows, A.col)
    uk, inv = np.unique(key, return_inverse=True)
    dv = rng.standard_normal(uk.shape[0])[inv]
    db = rng.standard_normal(A.n_rows)

    def loss(vals, bb):
        x = O.cg(A, bb, rtol=1e-14, vals=vals)["x"]
        return float(np.sum((x - t) ** 2))

    r = O.cg(A, b, rtol=1e-14)
    g = 2.0 * (r["x"] - t)
    bw = O.solve_backward(A, r["x"], g, symmetric=True, rtol=1e-14)
    analytic = float(bw["gvals"] @ dv + bw["lam"] @ db)
    for h in (1e-5, 1e-6):
        fd = (loss(A.vals + h * dv, b + h * db) - loss(A.vals - h * dv, b - h * db)) / (2 * h)
        assert abs(fd - analytic) <= 1e-5 * abs(analytic)


def test_adjoint_entrywise_fd_nonsymmetric_orientation():
    # Treat every stored value as an independent parameter: perturb single
    # off-diagonal entries (A stops being symmetric) and evaluate x = A^-1 b by
    # dense LU.  This pins the orientation -lambda_i x_j, which symmetric
    # directions cannot distinguish from -lambda_j x_i.
    N = 6
    A = W.varcoef_poisson5(N, seed=9)[0]
    b = W.rhs_uniform(A.n_rows, 3)
    t = np.random.default_rng(2).uniform(0, 1, A.n_rows)
    r = O.cg(A, b, rtol=1e-14)
    bw = O.solve_backward(A, r["x"], 2 * (r["x"] - t), symmetric=True, rtol=1e-14)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr))
    ks = [k for k in range(A.nnz) if rows[k] != A.col[k]][:12]
    for k in ks:
        def loss(h):
            v = A.vals.copy()
            v[k] += h
            x = np.linalg.solve(dense(A, v), b)
            return float(np.sum((x - t) ** 2))
        h = 1e-6
        fd = (loss(h) - loss(-h)) / (2 * h)
        assert abs(fd - bw["gvals"][k]) <= 1e-5 * max(abs(fd), 1e-3 * np.max(np.abs(bw["gvals"])))


def test_adjoint_matches_unrolled_reverse_mode():
    """The pages' naive path (paperpeel section 4.2): backpropagating through the CG
    iterations themselves, an O(k)-node graph built from a scatter-based SpMV
    (val * x[col], index_add).  Once the iteration has converged it must give the
    adjoint's gradients (with respect to A: along symmetric perturbations).  torch autograd on the CPU in float64, 16 x 16 variable-
    coefficient grid, the same number of iterations as the oracle's solve to 1e-14."""
    torch = pytest.importorskip("torch")
    A, b, _ = W.varcoef_poisson5(16, seed=7)
    f = O.cg(A, b, rtol=1e-14)
    assert f["state"] == O.CONVERGED
    K = f["iterations"]
    rows = torch.from_numpy(np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64))))
    cols = torch.from_numpy(A.col.astype(np.int64))
    vals = torch.tensor(A.vals, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)

    def spmv(p):
        return torch.zeros(A.n_rows, dtype=torch.float64).index_add(0, rows, vals * p[cols])

    x = torch.zeros(A.n_rows, dtype=torch.float64)
    r = bt.clone()
    p = r.clone()
    rho = r @ r
    for _ in range(K):
        q = spmv(p)
        alpha = rho / (p @ q)
        x = x + alpha * p
        r = r - alpha * q
        rho1 = r @ r
        p = r + (rho1 / rho) * p
        rho = rho1
    loss = 0.5 * (x @ x)
    loss.backward()
    bw = O.solve_backward(A, f["x"], f["x"], symmetric=True, rtol=1e-14)
    assert abs(loss.item() - 0.5 * float(f["x"] @ f["x"])) <= 1e-13 * loss.item()
    assert rel_err(bt.grad.numpy(), bw["lam"]) <= 1e-9
    # CG's recurrence assumes A = A^T, so its derivative along one stored entry alone (a
    # nonsymmetric perturbation) is not that of A^-1 b -- the pages see the same 1e-4
    # gap on the matrix gradient.  Along symmetric perturbations both are derivatives
    # of A^-1 b: the sums over each mirrored pair (i, j), (j, i) must agree.
    _, _, mirror = O.transpose(A)          # entry of A^T at position e = entry (j, i) of A
    sym_unrolled = vals.grad.numpy() + vals.grad.numpy()[mirror]
    sym_adjoint = bw["gvals"] + bw["gvals"][mirror]
    assert rel_err(sym_unrolled, sym_adjoint) <= 1e-9
    # while the single-entry values differ at the pages' level
    assert rel_err(vals.grad.numpy(), bw["gvals"]) <= 1e-2


def test_matvec_backward_against_dense():
    rng = np.random.default_rng(6)
    A = W.poisson5(7)
    vals = rng.standard_normal(A.nnz)
    x, gy = rng.standard_normal(A.n_cols), rng.standard_normal(A.n_rows)
    gx, gv = O.matvec_backward(A, x, gy, vals=vals)
    D = dense(A, vals)
    assert np.allclose(gx, D.T @ gy, rtol=0, atol=1e-13)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr))
    assert np.array_equal(gv, gy[rows] * x[A.col])
    # directional FD of L = <w, A x> in x and in vals (L is linear in each: exact up to rounding)
    w = gy
    dx = rng.standard_normal(A.n_cols)
    dvv = rng.standard_normal(A.nnz)
    fdx = (w @ (D @ (x + dx)) - w @ (D @ (x - dx))) / 2
    assert abs(fdx - gx @ dx) <= 1e-12 * (abs(w) @ abs(D) @ abs(dx))
    Dp, Dm = dense(A, vals + dvv), dense(A, vals - dvv)
    fdv = (w @ (Dp @ x) - w @ (Dm @ x)) / 2
    assert abs(fdv - gv @ dvv) <= 1e-12 * (np.abs(gv) @ np.abs(dvv))


# ----------------------------------------------------------------------------- transpose
def test_transpose_properties():
    rng = np.random.default_rng(12)
    # a rectangular, irregular pattern with empty rows and columns
    M = sp.random(37, 53, density=0.08, random_state=np.random.RandomState(1), format="csr")
    M.sort_indices()
    M.data = rng.standard_normal(M.nnz)
    A = W.CSR(37, 53, M.indptr.astype(np.int64), M.indices.astype(np.int32), M.data)
    rpt, ct, perm = O.transpose(A)
    T = M.T.tocsr()
    T.sort_indices()
    assert np.array_equal(rpt, T.indptr) and np.array_equal(ct, T.indices)
    assert np.array_equal(A.vals[perm], T.data)
    At = W.CSR(53, 37, rpt, ct, A.vals[perm])
    rpp, cc, pp = O.transpose(At)
    assert np.array_equal(rpp, A.row_ptr) and np.array_equal(cc, A.col)
    assert np.array_equal(perm[pp], np.arange(A.nnz))
    P = W.poisson5(9)
    rpt, ct, perm = O.transpose(P)
    assert np.array_equal(rpt, P.row_ptr) and np.array_equal(ct, P.col)
    assert np.array_equal(P.vals[perm], P.vals)


# ----------------------------------------------------------------------------- generators
def test_fem_generator_invariants():
    A, b = W.fem_p1_batched(nv=30, B=3, seed=4, mass=0.0)
    ones = np.ones(A.n_rows)
    for s in range(3):
        Ks = sp.csr_matrix((A.vals[s], A.col, A.row_ptr), shape=(A.n_rows,) * 2)
        assert np.max(np.abs(Ks @ ones)) <= 1e-12 * np.max(np.abs(A.vals[s]))
        assert abs(Ks - Ks.T).max() == 0.0
    Am, _ = W.fem_p1_batched(nv=30, B=1, seed=4, mass=1e-3, kappa_range=(1.0, 1.0))
    xy, tris = W._tri_mesh(30, np.random.default_rng(4), 0.3)
    P = xy[tris]
    area = 0.5 * np.abs((P[:, 1, 0] - P[:, 0, 0]) * (P[:, 2, 1] - P[:, 0, 1])
                        - (P[:, 1, 1] - P[:, 0, 1]) * (P[:, 2, 0] - P[:, 0, 0]))
    tot = float(Am.vals[0].sum())
    assert abs(tot - 1e-3 * area.sum()) <= 1e-12
    assert abs(area.sum() - 1.0) < 1e-2
    # nnz = n + 2 * edges for the diagonal-split structured mesh
    nv = 30
    edges = 2 * nv * (nv - 1) + (nv - 1) ** 2
    assert A.nnz == nv * nv + 2 * edges


def test_varcoef_reduces_to_poisson_when_kappa_is_one():
    N = 13
    V, b, _ = W.varcoef_poisson5(N, seed=0, kappa=np.ones((N + 2, N + 2)))
    P = W.poisson5(N)
    assert np.array_equal(V.row_ptr, P.row_ptr) and np.array_equal(V.col, P.col)
    assert np.array_equal(V.vals, P.vals)


def test_grf_marginal_variance():
    rng = np.random.default_rng(0)
    g = np.stack([W.gaussian_random_field(66, 1 / 65, 0.1, 1.0, rng) for _ in range(40)])
    var = float(np.mean(g ** 2))
    assert 0.8 < var < 1.2


def test_graph_laplacian_generator_invariants():
    # L + I of a weighted power-law graph: symmetric, every row sums to 1, columns
    # strictly ascending, positive definite (smallest eigenvalue 1: L 1 = 0), and the
    # row lengths skewed (hubs far above the median)
    A = W.graph_laplacian(3000, avg_deg=10.0, gamma=2.1, seed=5)
    M = sp.csr_matrix((A.vals, A.col, A.row_ptr), shape=(A.n_rows,) * 2)
    assert abs(M - M.T).max() == 0.0
    assert np.max(np.abs(M @ np.ones(A.n_rows) - 1.0)) <= 1e-12 * np.max(np.abs(A.vals))
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))
    same_row = rows[1:] == rows[:-1]
    assert np.all(A.col[1:][same_row] > A.col[:-1][same_row])
    lens = np.diff(A.row_ptr.astype(np.int64))
    assert lens.max() >= 30 * np.median(lens)
    off = A.vals[A.col != rows]
    assert np.all((off <= -0.5) & (off >= -1.5))
    small = W.graph_laplacian(300, avg_deg=6.0, gamma=2.1, seed=2)
    D = sp.csr_matrix((small.vals, small.col, small.row_ptr), shape=(300, 300)).toarray()
    ev = np.linalg.eigvalsh(D)
    assert abs(ev[0] - 1.0) <= 1e-12 * ev[-1] and ev[-1] <= 2.0 * np.max(np.diag(D)) + 1.0


def test_cg_and_adjoint_vs_dense_lu_on_a_graph_laplacian():
    # the skewed pattern through the oracle: CG and the adjoint against dense solves
    A = W.graph_laplacian(400, avg_deg=8.0, gamma=2.1, seed=3)
    D = sp.csr_matrix((A.vals, A.col, A.row_ptr), shape=(400, 400)).toarray()
    b = W.rhs_normal(400, 1)
    f = O.cg(A, b, rtol=1e-12)
    x = np.linalg.solve(D, b)
    assert f["state"] == O.CONVERGED
    kappa = np.linalg.cond(D)
    assert np.linalg.norm(f["x"] - x) <= kappa * 1e-12 * np.linalg.norm(x)
    bw = O.solve_backward(A, f["x"], f["x"], symmetric=True, rtol=1e-12)
    lam = np.linalg.solve(D.T, f["x"])
    assert np.linalg.norm(bw["lam"] - lam) <= kappa * 1e-12 * np.linalg.norm(lam)
    rows = np.repeat(np.arange(400), np.diff(A.row_ptr.astype(np.int64)))
    assert np.allclose(bw["gvals"], -lam[rows] * f["x"][A.col], rtol=1e-9, atol=1e-12 * np.abs(lam).max())
