"""GPU parity of the Jacobi-preconditioned CG (SLA_JACOBI), through the C ABI.

Against the oracle's orc_pcg_jacobi, with the bars of the plain solve: iterations
within 2 %, x within 1e-9, lambda and dL/dvals within 1e-8.  Every SpMV path is
covered: the fused plain kernel, the banded kernel and the split schedule (forced
through SLA_BAND_MIN_STRIDE / SLA_CG_SCHEDULE).  On the constant-diagonal Poisson
matrix Jacobi only rescales by a power of two, so the GPU's preconditioned iterates
must equal its plain ones bit for bit; a missing, non-positive or NaN diagonal entry
stops a system before its first iteration, after a zero right-hand side.
"""
import math

import numpy as np
import pytest

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


@pytest.fixture(params=["fused", "band", "split"])
def path(request, monkeypatch):
    monkeypatch.delenv("SLA_CG_SCHEDULE", raising=False)
    monkeypatch.delenv("SLA_BAND_MIN_STRIDE", raising=False)
    if request.param == "band":
        monkeypatch.setenv("SLA_BAND_MIN_STRIDE", "1")
    elif request.param == "split":
        monkeypatch.setenv("SLA_CG_SCHEDULE", "split")
    else:
        monkeypatch.setenv("SLA_CG_SCHEDULE", "fused")
    return request.param


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def iters_close(k_gpu, k_orc):
    return abs(k_gpu - k_orc) <= math.floor(0.02 * k_orc)


def handle(S, A):
    return S.csr_create(dev(A.row_ptr.astype(np.int32)), dev(A.col.astype(np.int32)), n_cols=A.n_cols,
                        symmetric=True)


def expect_path(S, h, path):
    an = S.csr_analysis(h)
    if path == "band":
        assert an["band_stride"] > 0
    elif path == "split":
        assert an["split"] and an["band_stride"] == 0
    else:
        assert not an["split"] and an["band_stride"] == 0


def solve(S, h, vals, b, jacobi, rtol=1e-10, max_iter=100000, fixed=False, hist=None):
    opts = S.cg_opts(rtol=rtol, max_iter=max_iter, fixed=fixed, jacobi=jacobi, residual_history=hist)
    x, info = S.solve(h, dev(vals), dev(b), opts)
    return x, S.read_info(info)


def test_jacobi_equals_plain_cg_bit_for_bit_on_poisson(S, path):
    A = W.poisson5(300)
    b = W.rhs_normal(A.n_rows, 3)
    h = handle(S, A)
    expect_path(S, h, path)
    K = 200
    h1 = torch.full((K + 1,), float("nan"), dtype=torch.float64, device="cuda")
    h2 = torch.full((K + 1,), float("nan"), dtype=torch.float64, device="cuda")
    x1, i1 = solve(S, h, A.vals, b, False, rtol=0.0, max_iter=K, fixed=True, hist=h1)
    x2, i2 = solve(S, h, A.vals, b, True, rtol=0.0, max_iter=K, fixed=True, hist=h2)
    assert i1[0]["iterations"] == i2[0]["iterations"] == K
    assert np.array_equal(host(x1), host(x2))
    assert np.array_equal(host(h1), host(h2))
    y1, j1 = solve(S, h, A.vals, b, False)
    y2, j2 = solve(S, h, A.vals, b, True)
    assert j1[0]["iterations"] == j2[0]["iterations"] and np.array_equal(host(y1), host(y2))


def check_pcg(S, h, A, vals, b, rtol=1e-10):
    """GPU PCG solve + adjoint (L = 0.5 |x|^2) against the oracle's, per system."""
    B = vals.shape[0]
    opts = S.cg_opts(rtol=rtol, jacobi=True)
    dv = dev(vals)
    x, info = S.solve(h, dv, dev(b), opts)
    gb, gv, binfo = S.solve_backward(h, dv, x, x.clone(), opts)
    xg, lam, gvals = host(x).reshape(B, -1), host(gb).reshape(B, -1), host(gv).reshape(B, -1)
    info, binfo = S.read_info(info), S.read_info(binfo)
    for s in range(B):
        f = O.cg(A, b[s], rtol=rtol, vals=vals[s], jacobi=True)
        assert info[s]["state"] == f["state"] == O.CONVERGED, (s, info[s], f["state"])
        assert iters_close(info[s]["iterations"], f["iterations"]), (s, info[s]["iterations"], f["iterations"])
        assert rel(xg[s], f["x"]) <= 1e-9, (s, rel(xg[s], f["x"]))
        bw = O.solve_backward(A, xg[s], xg[s], symmetric=True, rtol=rtol, vals=vals[s], jacobi=True)
        assert iters_close(binfo[s]["iterations"], bw["iterations"])
        assert rel(lam[s], bw["lam"]) <= 1e-8, (s, rel(lam[s], bw["lam"]))
        assert rel(gvals[s], bw["gvals"]) <= 1e-8
    return info


def test_jacobi_varcoef_against_oracle(S, path):
    N = 300                          # S = 300 admits the banded kernel when forced
    A, b, _ = W.varcoef_poisson5(N, seed=1)
    h = handle(S, A)
    expect_path(S, h, path)
    info = check_pcg(S, h, A, A.vals.reshape(1, -1), b.reshape(1, -1), rtol=1e-8)
    # the coefficient jumps make Jacobi pay
    plain = O.cg(A, b, rtol=1e-8)
    assert info[0]["iterations"] < 0.8 * plain["iterations"]


@pytest.mark.parametrize("grouped", ["1", "0"])
def test_jacobi_fem_batch_against_oracle(S, monkeypatch, grouped):
    # 16 systems on the split schedule: the grouped kernels (4 systems interleaved per
    # element), or the per-system ones with grouping switched off
    monkeypatch.setenv("SLA_CG_SCHEDULE", "split")
    monkeypatch.setenv("SLA_CG_GROUPED", grouped)
    A, b = W.fem_p1_batched(nv=24, B=16, seed=3)
    h = handle(S, A)
    check_pcg(S, h, A, A.vals, b, rtol=1e-8)


def test_jacobi_grouped_invalid_diagonals_and_agreement(S, monkeypatch):
    monkeypatch.setenv("SLA_CG_SCHEDULE", "split")
    A, b = W.fem_p1_batched(nv=24, B=8, seed=4)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))
    diag = np.nonzero(rows == A.col)[0]
    vals = A.vals.copy()
    b = b.copy()
    vals[1][diag[40]] = 0.0
    vals[2][diag[7]] = np.nan
    vals[3][diag[A.n_rows - 1]] = -2.0
    b[4] = 0.0
    h = handle(S, A)
    x, info = solve(S, h, vals, b, True, rtol=1e-8)
    inf = [i["state"] for i in info]
    assert inf[1:5] == [O.NOT_SPD, O.NAN, O.NOT_SPD, O.CONVERGED]
    xs = host(x).reshape(8, -1)
    for s_ in range(8):
        f = O.cg(A, b[s_], rtol=1e-8, vals=vals[s_], jacobi=True)
        assert info[s_]["state"] == f["state"], (s_, info[s_], f["state"])
        if f["state"] == O.CONVERGED:
            assert iters_close(info[s_]["iterations"], f["iterations"])
            assert rel(xs[s_], f["x"]) <= 1e-9, s_
    # grouped vs per-system kernels over 6 fixed iterations (system 0)
    xg, _ = solve(S, h, A.vals, b, True, rtol=0.0, max_iter=6, fixed=True)
    monkeypatch.setenv("SLA_CG_GROUPED", "0")
    h2 = handle(S, A)
    xu, _ = solve(S, h2, A.vals, b, True, rtol=0.0, max_iter=6, fixed=True)
    assert rel(host(xg), host(xu)) <= 1e-12


def test_jacobi_invalid_diagonals(S, path):
    A = W.poisson5(300)
    n = A.n_rows
    h = handle(S, A)
    rows = np.repeat(np.arange(n), np.diff(A.row_ptr.astype(np.int64)))
    diag = np.nonzero(rows == A.col)[0]
    v_zero, v_nan, v_neg = A.vals.copy(), A.vals.copy(), A.vals.copy()
    v_zero[diag[777]] = 0.0
    v_nan[diag[12]] = np.nan
    v_neg[diag[n - 1]] = -1.0
    vals = np.stack([A.vals, v_zero, v_nan, v_neg, v_nan])
    b = np.stack([W.rhs_normal(n, s) for s in range(5)])
    b[4] = 0.0                       # zero right-hand side: converged before the diagonal test
    x, info = solve(S, h, vals, b, True, rtol=1e-8)
    states = [i["state"] for i in info]
    assert states == [O.CONVERGED, O.NOT_SPD, O.NAN, O.NOT_SPD, O.CONVERGED]
    assert all(info[s]["iterations"] == 0 for s in (1, 2, 3, 4))
    xs = host(x).reshape(5, n)
    assert not np.any(xs[1:])
    for s in (1, 2, 3):
        assert O.cg(A, b[s], rtol=1e-8, vals=vals[s], jacobi=True)["state"] == states[s]
    f = O.cg(A, b[0], rtol=1e-8, vals=vals[0], jacobi=True)
    assert rel(xs[0], f["x"]) <= 1e-9


def test_jacobi_autograd(S):
    A, b, _ = W.varcoef_poisson5(24, seed=6)
    T = S.SparseTensor(dev(A.row_ptr.astype(np.int32)), dev(A.col), dev(A.vals).requires_grad_(True),
                       symmetric=True)
    bt = dev(b).requires_grad_(True)
    x = T.solve(bt, rtol=1e-12, jacobi=True)
    (0.5 * (x * x).sum()).backward()
    f = O.cg(A, b, rtol=1e-12, jacobi=True)
    bw = O.solve_backward(A, host(x), host(x), symmetric=True, rtol=1e-12, jacobi=True)
    assert rel(host(x), f["x"]) <= 1e-9
    assert rel(host(bt.grad), bw["lam"]) <= 1e-8
    assert rel(host(T.vals.grad), bw["gvals"]) <= 1e-8
