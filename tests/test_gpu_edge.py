"""Degenerate inputs through the C ABI, against the oracle: a 0 x 0 matrix (matvec,
solve and the adjoint are empty and converged with 0 iterations; the eigensolvers
refuse it), a pattern with no stored entries (A = 0: y = 0, NOT_SPD for b != 0,
converged with 0 iterations for b = 0, an empty gradient), and a 1 x 1 system (one
CG iteration, exact)."""
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


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t if dtype is None else t.to(dtype)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def handle(S, A, symmetric=True):
    return S.csr_create(dev(A.row_ptr.astype(np.int32)), dev(A.col.astype(np.int32)), n_cols=A.n_cols,
                        symmetric=symmetric)


def test_empty_matrix(S):
    A = W.CSR(0, 0, np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0))
    h = handle(S, A)
    vals = dev(A.vals)
    y = S.matvec(h, vals, dev(np.zeros(0)))
    assert host(y).shape == (0,)
    for sym in (True, False):
        h = handle(S, A, symmetric=sym)
        x, info = S.solve(h, vals, dev(np.zeros(0)), S.cg_opts(rtol=1e-8))
        gb, gv, binfo = S.solve_backward(h, vals, x, x.clone(), S.cg_opts(rtol=1e-8))
        f = O.cg(A, np.zeros(0), rtol=1e-8)
        for inf in (S.read_info(info)[0], S.read_info(binfo)[0]):
            assert inf["state"] == f["state"] == O.CONVERGED and inf["iterations"] == f["iterations"] == 0
        assert host(x).shape == host(gb).shape == host(gv).shape == (0,)
    with pytest.raises(S.SlaError):
        S.eigsh(handle(S, A), vals, 1, dev(np.zeros(0)))


def test_pattern_without_entries(S):
    n = 300
    A = W.CSR(n, n, np.zeros(n + 1, np.int32), np.zeros(0, np.int32), np.zeros(0))
    vals = dev(A.vals)
    for sym in (True, False):
        h = handle(S, A, symmetric=sym)
        y = S.matvec(h, vals, dev(np.arange(1.0, n + 1.0)))
        assert np.array_equal(host(y), O.spmv(A, np.arange(1.0, n + 1.0)))
        b = W.rhs_normal(n, 1)
        x, info = S.solve(h, vals, dev(b), S.cg_opts(rtol=1e-8))
        f = O.cg(A, b, rtol=1e-8)
        inf = S.read_info(info)[0]
        assert inf["state"] == f["state"] == O.NOT_SPD and inf["iterations"] == f["iterations"] == 0
        x0, info0 = S.solve(h, vals, dev(np.zeros(n)), S.cg_opts(rtol=1e-8))
        i0 = S.read_info(info0)[0]
        assert i0["state"] == O.CONVERGED and i0["iterations"] == 0 and not np.any(host(x0))
        gb, gv, binfo = S.solve_backward(h, vals, x0, x0.clone(), S.cg_opts(rtol=1e-8))
        assert S.read_info(binfo)[0]["state"] == O.CONVERGED and host(gv).shape == (0,)


def test_one_by_one(S):
    A = W.CSR(1, 1, np.array([0, 1], np.int32), np.array([0], np.int32), np.array([4.0]))
    h = handle(S, A)
    x, info = S.solve(h, dev(A.vals), dev(np.array([2.0])), S.cg_opts(rtol=1e-12))
    gb, gv, binfo = S.solve_backward(h, dev(A.vals), x, torch.ones_like(x), S.cg_opts(rtol=1e-12))
    f = O.cg(A, np.array([2.0]), rtol=1e-12)
    bw = O.solve_backward(A, f["x"], np.ones(1), symmetric=True, rtol=1e-12)
    assert S.read_info(info)[0]["iterations"] == f["iterations"] == 1
    assert host(x)[0] == f["x"][0] == 0.5
    assert host(gb)[0] == bw["lam"][0] == 0.25 and host(gv)[0] == bw["gvals"][0] == -0.125
