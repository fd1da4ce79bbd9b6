"""GPU parity of the Lanczos eigensolver (sla_eigsh) and of the Hellmann-Feynman
eigenvalue gradient (sla_eigsh_backward), through the C ABI.

The reference is the oracle's Lanczos (oracle/eigsh.py): the same steps, the same stop
test after every step, the same start vector.  Converged Ritz pairs do not depend on
the rounding of the steps beyond what the stop test allows: eigenvalue errors are of
order (tol theta)^2 / gap and eigenvector errors of order tol theta / gap.  Bars:
eigenvalues within 1e-12 |A| (Weyl: rounding perturbs an eigenvalue by a multiple of
eps |A| whatever its size, so the smallest ones are held to the spectrum's scale), unit
eigenvectors (both signed by <u, v0> >= 0) within 1e-7, the Krylov dimension at the
stop within 2 steps of the oracle's, and the gradient within 1e-7 of the oracle's on the oracle's vectors and bit for bit on the
GPU's own vectors (same products, same order).  With thick restart (a basis of
max_dim vectors restarted until max_iter steps) the stop test runs once per cycle, so
the bar on the step count becomes the same number of restarts and steps as the oracle.
"""
import math

import numpy as np
import pytest
import scipy.sparse as sp

import oracle as O
import workloads as W
from oracle.eigsh import eigsh as orc_eigsh, eigsh_grad as orc_eigsh_grad

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


def handle(S, A, symmetric=True):
    return S.csr_create(dev(A.row_ptr.astype(np.int32)), dev(A.col.astype(np.int32)), n_cols=A.n_cols,
                        symmetric=symmetric)


def csr_of_dense(M):
    Sm = sp.csr_matrix(M)
    Sm.sort_indices()
    return W.CSR(M.shape[0], M.shape[1], Sm.indptr.astype(np.int32), Sm.indices.astype(np.int32),
                 Sm.data.astype(np.float64))


def norm_inf(A):
    """Largest absolute row sum: a bound on |A|_2, the scale of eigenvalue rounding."""
    return float(np.add.reduceat(np.abs(A.vals), A.row_ptr[:-1].astype(np.int64)).max())


def compare(S, A, k, which, tol, seed=1, g=None, max_dim=0, max_iter=0, keep=0):
    v0 = W.rhs_normal(A.n_rows, seed)
    h = handle(S, A)
    ev, U, info = S.eigsh(h, dev(A.vals), k, dev(v0), which=which, tol=tol, max_dim=max_dim, max_iter=max_iter,
                          keep=keep)
    ev, U = host(ev), host(U)
    r = orc_eigsh(A, k, v0, which=which, tol=tol, max_dim=max_dim or None, max_iter=max_iter or None,
                  keep=keep or None)
    assert info["state"] == r["state"], (info, r["state"])
    if r["restarts"] == 0:
        assert info["restarts"] == 0
        assert abs(info["iterations"] - r["iterations"]) <= 2, (info["iterations"], r["iterations"])
    else:
        # with restarts the stop test runs once per cycle: the same cycle (the cases keep
        # the deciding residuals well away from tol, so rounding cannot move the stop)
        assert (info["restarts"], info["iterations"]) == (r["restarts"], r["iterations"]), (info, r["restarts"],
                                                                                            r["iterations"])
    scale = max(np.abs(r["evals"]).max(), norm_inf(A))
    assert np.abs(ev - r["evals"]).max() <= 1e-12 * scale, np.abs(ev - r["evals"]).max() / scale
    for i in range(k):
        assert abs(np.linalg.norm(U[i]) - 1.0) <= 1e-13
        assert U[i] @ v0 >= 0.0
        assert np.linalg.norm(U[i] - r["evecs"][i]) <= 1e-7, (i, np.linalg.norm(U[i] - r["evecs"][i]))
    if g is not None:
        gv = host(S.eigsh_backward(h, dev(U), dev(g)))
        ref = orc_eigsh_grad(A, r["evecs"], g)
        assert np.linalg.norm(gv - ref) <= 1e-7 * np.linalg.norm(ref)
        assert np.array_equal(gv, orc_eigsh_grad(A, U, g))
    return ev, U, info, r


@pytest.mark.parametrize("which", ["largest", "smallest"])
def test_eigsh_varcoef_small(S, which):
    A, _, _ = W.varcoef_poisson5(40, seed=1)
    compare(S, A, 4, which, 1e-10, g=np.array([1.0, -0.5, 2.0, 0.25]))


def test_eigsh_varcoef_300(S):
    # 90,000 rows: 352 tiles with a ragged last one, 88 reorthogonalization workgroups
    A, _, _ = W.varcoef_poisson5(300, seed=2)
    ev, U, info, r = compare(S, A, 6, "largest", 1e-10, seed=3, g=np.linspace(1.0, 2.0, 6))
    assert info["iterations"] > 20


def test_eigsh_laplacian_closed_form(S):
    nx, ny = 120, 97
    Tx = sp.diags([-1.0, 2.0, -1.0], [-1, 0, 1], shape=(nx, nx))
    Ty = sp.diags([-1.0, 2.0, -1.0], [-1, 0, 1], shape=(ny, ny))
    A = csr_of_dense((sp.kron(sp.eye(ny), Tx) + sp.kron(Ty, sp.eye(nx))).toarray())
    lam = np.sort([4 - 2 * math.cos(p * math.pi / (nx + 1)) - 2 * math.cos(q * math.pi / (ny + 1))
                   for p in range(1, nx + 1) for q in range(1, ny + 1)])[::-1][:3]
    h = handle(S, A)
    ev, U, info = S.eigsh(h, dev(A.vals), 3, dev(W.rhs_normal(A.n_rows, 5)), which="largest", tol=1e-11)
    assert info["state"] == O.CONVERGED
    assert np.abs(host(ev) - lam).max() <= 1e-12 * lam[0]


def test_eigsh_invariant_subspace_and_breakdown(S):
    n = 5000
    A = W.CSR(n, n, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32), np.arange(1.0, n + 1.0))
    v0 = np.zeros(n)
    v0[[6, 4031]] = [3.0, -2.0]
    h = handle(S, A)
    ev, U, info = S.eigsh(h, dev(A.vals), 2, dev(v0), which="largest", tol=1e-12)
    assert info["state"] == O.CONVERGED and info["iterations"] == 2
    assert np.abs(host(ev) - [4032.0, 7.0]).max() <= 1e-12 * 4032
    U = host(U)
    assert U[0][4031] < 0 and abs(U[0][4031] + 1.0) <= 1e-13 and abs(U[1][6] - 1.0) <= 1e-13
    _, _, info3 = S.eigsh(h, dev(A.vals), 3, dev(v0), which="largest", tol=1e-12)
    assert info3["state"] == O.BREAKDOWN and info3["iterations"] == 2


def test_eigsh_dimension_cap(S):
    A, _, _ = W.varcoef_poisson5(30, seed=4)
    # 12 steps from a fixed start: Ritz values of a fixed Krylov space (no stop point to
    # move), so the bars are those of the rounding alone
    compare(S, A, 3, "smallest", 1e-14, seed=3, max_dim=12)


@pytest.mark.parametrize("N,seed,k,which,tol,m", [
    (40, 1, 4, "smallest", 3e-11, 30),     # 93 restarts of a 30-vector basis
    (40, 1, 4, "largest", 1e-10, 20),
    (300, 2, 6, "largest", 1e-9, 40),      # 90,000 rows: 1,407 restart workgroups of 64 rows
    (120, 3, 8, "smallest", 1e-10, 200),   # 40 rows per restart workgroup
])
def test_eigsh_thick_restart(S, N, seed, k, which, tol, m):
    A, _, _ = W.varcoef_poisson5(N, seed=seed)
    g = np.linspace(-1.0, 1.0, k)
    ev, U, info, r = compare(S, A, k, which, tol, seed=3, g=g, max_dim=m, max_iter=200000)
    assert info["state"] == O.CONVERGED and info["restarts"] > 0


def test_eigsh_thick_restart_budget_and_keep(S):
    # the step budget ends mid-cycle (MAX_ITER with the Ritz pairs of that basis), with the
    # default keep and with keep = 10.  Unconverged Ritz values of a restarted Krylov
    # space are ill-conditioned functions of the rounding (Krylov subspaces are
    # exponentially sensitive to their start vector: Carpraux, Godunov and Kuznetsov,
    # 1996): the oracle itself moves them by 2.8e-7 and 4.9e-9 here when v0 is perturbed
    # by 1e-15.  So the counts are exact, the values match the oracle to 1e-5 |theta|,
    # and what every correct run satisfies is checked to rounding: the Lanczos relation
    # (the reported estimate is the true residual), Rayleigh quotients, and Cauchy
    # interlacing with the dense spectrum.
    A, _, _ = W.varcoef_poisson5(40, seed=1)
    v0 = W.rhs_normal(A.n_rows, 3)
    h = handle(S, A)
    M = sp.csr_matrix((A.vals, A.col, A.row_ptr.astype(np.int64)), shape=(A.n_rows, A.n_cols))
    lam = np.linalg.eigvalsh(M.toarray())
    nA = norm_inf(A)
    for max_iter, keep in [(30 + 3 * 17 + 5, 0), (30 + 2 * 20 + 7, 10)]:
        ev, U, info = S.eigsh(h, dev(A.vals), 4, dev(v0), which="smallest", tol=1e-12, max_dim=30,
                              max_iter=max_iter, keep=keep)
        r = orc_eigsh(A, 4, v0, which="smallest", tol=1e-12, max_dim=30, max_iter=max_iter, keep=keep or None)
        assert info["state"] == r["state"] == O.MAX_ITER
        assert info["iterations"] == r["iterations"] == max_iter
        assert info["restarts"] == r["restarts"] > 0
        ev, U = host(ev), host(U)
        assert np.all(np.abs(ev - r["evals"]) <= 1e-5 * np.abs(r["evals"]))
        assert np.allclose(U @ U.T, np.eye(4), atol=1e-12)
        res = np.array([np.linalg.norm(M @ U[i] - ev[i] * U[i]) for i in range(4)])
        assert abs(res.max() - info["max_res"]) <= 1e-10 * nA
        for i in range(4):
            assert abs(U[i] @ (M @ U[i]) - ev[i]) <= 1e-12 * nA
            assert ev[i] >= lam[i] - 1e-12 * nA     # the i-th Ritz value from below


def test_eigsh_argument_errors(S):
    A, _, _ = W.varcoef_poisson5(10, seed=1)
    v0 = dev(W.rhs_normal(A.n_rows, 1))
    with pytest.raises(S.SlaError):          # Lanczos needs a symmetric handle
        S.eigsh(handle(S, A, symmetric=False), dev(A.vals), 2, v0)
    h = handle(S, A)
    with pytest.raises(S.SlaError):
        S.eigsh(h, dev(A.vals), 2, torch.zeros_like(v0))
    with pytest.raises(S.SlaError):
        S.eigsh(h, dev(A.vals), 33, v0)
    with pytest.raises(S.SlaError):
        S.eigsh(h, dev(A.vals), 5, v0, max_dim=4)
    with pytest.raises(S.SlaError):          # keep must lie in [k, max_dim)
        S.eigsh(h, dev(A.vals), 3, v0, max_dim=10, max_iter=50, keep=10)
    with pytest.raises(S.SlaError):
        S.eigsh(h, dev(A.vals), 3, v0, max_dim=10, max_iter=50, keep=2)
    with pytest.raises(S.SlaError):          # max_dim = k leaves nothing to restart with
        S.eigsh(h, dev(A.vals), 3, v0, max_dim=3, max_iter=50)
    Abig, _, _ = W.varcoef_poisson5(40, seed=1)
    with pytest.raises(S.SlaError):          # basis cap with restart
        S.eigsh(handle(S, Abig), dev(Abig.vals), 3, dev(W.rhs_normal(Abig.n_rows, 1)), max_dim=1025, max_iter=5000)


def test_eigsh_autograd_thick_restart(S):
    A, _, _ = W.varcoef_poisson5(24, seed=6)
    v0 = W.rhs_normal(A.n_rows, 2)
    T = S.SparseTensor(dev(A.row_ptr.astype(np.int32)), dev(A.col), dev(A.vals).requires_grad_(True),
                       symmetric=True)
    ev, U = T.eigsh(k=2, which="largest", tol=1e-12, v0=dev(v0), max_dim=12, max_iter=5000)
    assert T.last_eig_info["restarts"] > 0
    (ev * torch.tensor([1.0, -3.0], dtype=torch.float64, device="cuda")).sum().backward()
    r = orc_eigsh(A, 2, v0, which="largest", tol=1e-12, max_dim=12, max_iter=5000)
    ref = orc_eigsh_grad(A, r["evecs"], np.array([1.0, -3.0]))
    assert np.linalg.norm(host(T.vals.grad) - ref) <= 1e-7 * np.linalg.norm(ref)


def test_eigsh_autograd(S):
    A, _, _ = W.varcoef_poisson5(24, seed=6)
    v0 = W.rhs_normal(A.n_rows, 2)
    T = S.SparseTensor(dev(A.row_ptr.astype(np.int32)), dev(A.col), dev(A.vals).requires_grad_(True),
                       symmetric=True)
    ev, U = T.eigsh(k=3, which="smallest", tol=1e-12, v0=dev(v0))
    assert not U.requires_grad
    w = torch.tensor([1.0, 2.0, -1.0], dtype=torch.float64, device="cuda")
    (w * ev).sum().backward()
    r = orc_eigsh(A, 3, v0, which="smallest", tol=1e-12)
    ref = orc_eigsh_grad(A, r["evecs"], np.array([1.0, 2.0, -1.0]))
    assert np.linalg.norm(host(T.vals.grad) - ref) <= 1e-7 * np.linalg.norm(ref)


def test_eigsh_k32(S):
    # the most Ritz vectors a call returns (k_lz_ritz with 32 accumulators)
    A, _, _ = W.varcoef_poisson5(30, seed=8)
    compare(S, A, 32, "largest", 1e-10, seed=100, g=np.linspace(-1.0, 1.0, 32))
