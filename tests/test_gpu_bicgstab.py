"""GPU parity of BiCGStab (SLA_BICGSTAB) and its adjoint on A^T, through the C ABI.

BiCGStab (van der Vorst, 1992) is the pages' iterative method for nonsymmetric
systems (torch-sla, paperpeel page, sections 1 and 3.1).  The reference is the
oracle's orc_bicgstab.

Bars.  BiCGStab's iterates amplify rounding far more than CG's on ill-conditioned
systems.  On the CPU, two runs that differ only in the summation order of their inner
products give:
  * the same iterates to 7e-15 over the first 12 iterations of an unshifted 300 x 300
    convection-diffusion system (2e-13 after 16);
  * stop points up to 13 % apart (Poisson 300 x 300 at rtol 1e-8: 584, 632 and 661
    iterations) and solutions 1e-6 apart, all of them meeting the stop test;
  * on shifted systems (a reaction term c = 1), identical counts and solutions to 1e-15.
Accordingly:
  - well-conditioned (shifted) systems carry CG's bars: iterations within 2 %, x
    within 1e-9, lambda and dL/dvals within 1e-8;
  - fixed runs of 10 iterations: x and the residual history within 1e-12;
  - ill-conditioned systems are held to what the stop test fixes: both solutions
    satisfy |b - A x| <= rtol |b| up to the drift of the recurrence residual, so
    |A (x_gpu - x_oracle)| <= 3 rtol |b| and the GPU's true residual <= 2 rtol |b|
    (and the same for lambda with A^T); dL/dvals = -lambda_i x_j is then checked bit
    for bit on the GPU's own lambda and x; iteration counts within 20 %.
"""
import math

import numpy as np
import pytest
import scipy.sparse as sp

import oracle as O
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differentiable_sparse_linear_spmv_amd as S
    return S


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def iters_close(k_gpu, k_orc, bar=0.02):
    return abs(k_gpu - k_orc) <= math.floor(bar * k_orc)


def handle(S, A, symmetric=False):
    return S.csr_create(dev(A.row_ptr.astype(np.int32)), dev(A.col.astype(np.int32)), n_cols=A.n_cols,
                        symmetric=symmetric)


def spm(A, vals):
    return sp.csr_matrix((vals, A.col, A.row_ptr.astype(np.int64)), shape=(A.n_rows, A.n_cols))


def gpu_pair(S, h, vals, b, rtol, max_iter=100000, fixed=False, hist=None):
    """GPU BiCGStab solve, then its adjoint for L = 0.5 |x|^2 per system."""
    opts = S.cg_opts(rtol=rtol, max_iter=max_iter, fixed=fixed, method="bicgstab", residual_history=hist)
    dv = dev(vals)
    x, info = S.solve(h, dv, dev(b), opts)
    gb, gv, binfo = S.solve_backward(h, dv, x, x.clone(), S.cg_opts(rtol=rtol, max_iter=max_iter, fixed=fixed,
                                                                     method="bicgstab"))
    B = vals.shape[0]
    return (host(x).reshape(B, -1), host(gb).reshape(B, -1), host(gv).reshape(B, -1), S.read_info(info),
            S.read_info(binfo))


def check_tight(A, vals, b, out, rtol, symmetric=False, systems=None, fixed=False, max_iter=100000):
    x, lam, gv, info, binfo = out
    tol_x, tol_adj = (1e-12, 1e-12) if fixed else (1e-9, 1e-8)
    for s in (range(vals.shape[0]) if systems is None else systems):
        f = O.bicgstab(A, b[s], rtol=rtol, vals=vals[s], fixed=fixed, max_iter=max_iter)
        assert info[s]["state"] == f["state"], (s, info[s], f["state"])
        assert iters_close(info[s]["iterations"], f["iterations"]), (s, info[s]["iterations"], f["iterations"])
        assert rel(x[s], f["x"]) <= tol_x, (s, rel(x[s], f["x"]))
        bw = O.solve_backward(A, x[s], x[s], symmetric=symmetric, rtol=rtol, vals=vals[s], method="bicgstab",
                              fixed=fixed, max_iter=max_iter)
        assert binfo[s]["state"] == bw["state"]
        assert iters_close(binfo[s]["iterations"], bw["iterations"]), (s, binfo[s]["iterations"],
                                                                       bw["iterations"])
        assert rel(lam[s], bw["lam"]) <= tol_adj, (s, rel(lam[s], bw["lam"]))
        assert rel(gv[s], bw["gvals"]) <= tol_adj, (s, rel(gv[s], bw["gvals"]))


def check_by_residual(A, vals, b, out, rtol, iter_bar=0.20):
    """Ill-conditioned systems: the bounds the stop test fixes (module docstring)."""
    x, lam, gv, info, binfo = out
    for s in range(vals.shape[0]):
        M = spm(A, vals[s])
        f = O.bicgstab(A, b[s], rtol=rtol, vals=vals[s])
        assert info[s]["state"] == f["state"] == O.CONVERGED, (s, info[s], f["state"])
        assert iters_close(info[s]["iterations"], f["iterations"], iter_bar), (s, info[s]["iterations"],
                                                                              f["iterations"])
        nb = np.linalg.norm(b[s])
        assert np.linalg.norm(O.spmv(A, x[s] - f["x"], vals=vals[s])) <= 3 * rtol * nb
        assert np.linalg.norm(b[s] - M @ x[s]) <= 2 * rtol * nb
        assert info[s]["rhs_norm"] == pytest.approx(nb, rel=1e-12)
        bw = O.solve_backward(A, x[s], x[s], symmetric=False, rtol=rtol, vals=vals[s], method="bicgstab")
        assert binfo[s]["state"] == bw["state"] == O.CONVERGED
        assert iters_close(binfo[s]["iterations"], bw["iterations"], iter_bar)
        ng = np.linalg.norm(x[s])
        assert np.linalg.norm(M.T @ (lam[s] - bw["lam"])) <= 3 * rtol * ng
        assert np.linalg.norm(x[s] - M.T @ lam[s]) <= 2 * rtol * ng
        # the gradient scatter is exact given lambda and x
        assert np.array_equal(gv[s], O.pattern_outer(A, lam[s], x[s], sign=-1.0))


# ------------------------------------------------------------------------- tight bars
def test_bicgstab_shifted_convdiff(S):
    # 300 x 300: 352 tiles with a ragged last one; nonsymmetric handle: the adjoint
    # runs BiCGStab on the device transpose
    A = W.convdiff5(300, wind=100.0, shift=1.0)
    b = W.rhs_normal(A.n_rows, 3).reshape(1, -1)
    out = gpu_pair(S, handle(S, A), A.vals.reshape(1, -1), b, rtol=1e-10)
    assert out[3][0]["iterations"] > 10
    check_tight(A, A.vals.reshape(1, -1), b, out, rtol=1e-10)


def test_bicgstab_batch_of_winds(S):
    # shared pattern, one wind per system (3 systems, then 8: every system on one XCD)
    for B in (3, 8):
        winds = [20.0 + 280.0 * s / (B - 1) for s in range(B)]
        A = W.convdiff5(200, wind=winds, shift=1.0)
        b = np.stack([W.rhs_normal(A.n_rows, 10 + s) for s in range(B)])
        out = gpu_pair(S, handle(S, A), A.vals, b, rtol=1e-10)
        check_tight(A, A.vals, b, out, rtol=1e-10, systems=[0, 1, B - 1])
        assert len({i["iterations"] for i in out[3]}) > 1     # systems stop independently


def test_bicgstab_fixed_iterations_and_history(S):
    A = W.convdiff5(300, wind=100.0)
    b = W.rhs_normal(A.n_rows, 4)
    K = 10
    hist = torch.full((K + 1,), float("nan"), dtype=torch.float64, device="cuda")
    out = gpu_pair(S, handle(S, A), A.vals.reshape(1, -1), b.reshape(1, -1), rtol=0.0, max_iter=K, fixed=True,
                   hist=hist)
    f = O.bicgstab(A, b, rtol=0.0, max_iter=K, fixed=True, history=True)
    assert out[3][0]["iterations"] == K and out[3][0]["state"] == O.MAX_ITER
    assert rel(host(hist), f["history"]) <= 1e-12
    check_tight(A, A.vals.reshape(1, -1), b.reshape(1, -1), out, rtol=0.0, fixed=True, max_iter=K)


def test_bicgstab_exact_cases(S):
    # 4 I: one iteration, stopped half-way with x = b / 4 (alpha = 1/4 up to the
    # rounding of two different reduction trees, so to a few units in the last place)
    n = 5000
    D = W.CSR(n, n, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32), np.full(n, 4.0))
    b = W.rhs_normal(n, 5)
    hist = torch.full((3,), float("nan"), dtype=torch.float64, device="cuda")
    out = gpu_pair(S, handle(S, D, symmetric=True), D.vals.reshape(1, -1), b.reshape(1, -1), rtol=1e-14,
                   max_iter=2, hist=hist)
    assert out[3][0]["iterations"] == 1 and out[3][0]["state"] == O.CONVERGED
    assert rel(out[0][0], b / 4.0) <= 4e-16
    h = host(hist)
    assert h[1] <= 1e-15 * np.linalg.norm(b) and np.isnan(h[2])
    # Laplacian eigenvector: one iteration, x = v / lambda
    N, p, q = 64, 3, 5
    A = W.poisson5(N)
    i = np.arange(1, N + 1)
    v = np.outer(np.sin(p * np.pi * i / (N + 1)), np.sin(q * np.pi * i / (N + 1))).reshape(-1)
    lam = 4.0 - 2.0 * math.cos(p * math.pi / (N + 1)) - 2.0 * math.cos(q * math.pi / (N + 1))
    out = gpu_pair(S, handle(S, A, symmetric=True), A.vals.reshape(1, -1), v.reshape(1, -1), rtol=1e-10)
    assert out[3][0]["iterations"] == 1
    assert rel(out[0][0], v / lam) <= 1e-13


def test_bicgstab_outcomes_in_one_batch(S):
    # pattern: diagonal plus the pairs (2j, 2j + 1); system 0 is a pure rotation
    # (<b, A b> = 0: BREAKDOWN at once), 1 is 2 I + rotation (converges), 2 holds a NaN,
    # 3 has b = 0 (converged, 0 iterations), 4 runs out of budget
    n = 4000
    rows, cols = [], []
    for j in range(0, n, 2):
        rows += [j, j, j + 1, j + 1]
        cols += [j, j + 1, j, j + 1]
    rows, cols = np.array(rows), np.array(cols)
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    rp = np.cumsum(rp).astype(np.int32)
    base_off = np.where(cols > rows, -1.0, np.where(cols < rows, 1.0, 0.0))
    diag = (cols == rows)
    spread = 1.0 + np.random.default_rng(7).uniform(0.0, 1.0, rows.shape[0])   # many distinct eigenvalues
    vals = np.stack([base_off, base_off + 2.0 * diag, base_off + 2.0 * diag, base_off + 2.0 * diag,
                     base_off + spread * diag])
    vals[2][17] = np.nan
    A = W.CSR(n, n, rp, cols.astype(np.int32), vals[1])
    b = np.stack([W.rhs_normal(n, 20 + s) for s in range(5)])
    b[3] = 0.0
    h = handle(S, A)
    opts = S.cg_opts(rtol=1e-12, max_iter=3, method="bicgstab")
    x, info = S.solve(h, dev(vals), dev(b), opts)
    inf = S.read_info(info)
    xs = host(x).reshape(5, n)
    for s in range(5):
        f = O.bicgstab(A, b[s], rtol=1e-12, max_iter=3, vals=vals[s])
        assert inf[s]["state"] == f["state"], (s, inf[s], f["state"])
        assert inf[s]["iterations"] == f["iterations"], (s, inf[s], f["iterations"])
        if f["state"] in (O.CONVERGED, O.MAX_ITER):
            assert rel(xs[s], f["x"]) <= 1e-12, s
    assert [i["state"] for i in inf] == [O.BREAKDOWN, O.CONVERGED, O.NAN, O.CONVERGED, O.MAX_ITER]
    assert not np.any(xs[0]) and not np.any(xs[3])


def test_bicgstab_flag_checks(S):
    A = W.convdiff5(20, wind=10.0)
    h = handle(S, A)
    with pytest.raises(S.SlaError):
        S.solve(h, dev(A.vals), dev(W.rhs_normal(A.n_rows, 1)),
                S.cg_opts(method="bicgstab", jacobi=True))


def test_bicgstab_autograd(S):
    A = W.convdiff5(30, wind=150.0, shift=1.0)
    b = W.rhs_normal(A.n_rows, 6)
    T = S.SparseTensor(dev(A.row_ptr.astype(np.int32)), dev(A.col), dev(A.vals).requires_grad_(True))
    bt = dev(b).requires_grad_(True)
    x = T.solve(bt, rtol=1e-12, method="bicgstab", check=True)
    (0.5 * (x * x).sum()).backward()
    f = O.bicgstab(A, b, rtol=1e-12)
    bw = O.solve_backward(A, host(x), host(x), symmetric=False, rtol=1e-12, method="bicgstab")
    assert rel(host(x), f["x"]) <= 1e-9
    assert rel(host(bt.grad), bw["lam"]) <= 1e-8
    assert rel(host(T.vals.grad), bw["gvals"]) <= 1e-8


# ------------------------------------------------------------- bars from the stop test
def test_bicgstab_unshifted_convdiff(S):
    A = W.convdiff5(300, wind=100.0)
    b = W.rhs_normal(A.n_rows, 4).reshape(1, -1)
    out = gpu_pair(S, handle(S, A), A.vals.reshape(1, -1), b, rtol=1e-8)
    check_by_residual(A, A.vals.reshape(1, -1), b, out, rtol=1e-8)


def test_bicgstab_fem_with_skew_part(S):
    # FEM pattern (permuted vertex ids: scattered columns), values made nonsymmetric by
    # +-0.3 |a_ij| on the upper / lower entries
    F, bf = W.fem_p1_batched(nv=60, B=2, seed=2)
    rows = np.repeat(np.arange(F.n_rows), np.diff(F.row_ptr.astype(np.int64)))
    skew = np.where(F.col > rows, 0.3, np.where(F.col < rows, -0.3, 0.0))
    vals = F.vals + skew * np.abs(F.vals)
    out = gpu_pair(S, handle(S, F), vals, bf, rtol=1e-10)
    check_by_residual(F, vals, bf, out, rtol=1e-10)
