"""GPU parity of SparseTensorList solves (sla_list_*): systems with distinct patterns
solved together, through the C ABI.

The pages' second batching mode (torch-sla, paperpeel page, section 3.1 "Typed
sparse-tensor hierarchy").  Each item must behave as the oracle's CG on that item
alone, with the bars of the single-system path: iterations within 2 %, x within 1e-9,
lambda and dL/dvals within 1e-8, fixed iterations within 1e-12.  Items of different
sizes share the grid (a Poisson grid with ragged tiles, a permuted FEM mesh, a
variable-coefficient grid, a one-row system, a 300 x 300 grid spanning many
workgroups), under both CG schedules.
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


@pytest.fixture(params=["fused", "split"])
def schedule(request, monkeypatch):
    monkeypatch.setenv("SLA_CG_SCHEDULE", request.param)
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


def items_mixed():
    """(CSR, vals, b) per item, distinct patterns and sizes."""
    out = []
    A = W.poisson5(40)                                      # 1600 rows: 6 tiles + 64
    out.append((A, A.vals, W.rhs_normal(A.n_rows, 1)))
    F, bf = W.fem_p1_batched(nv=30, B=1, seed=2)            # permuted mesh, 900 rows
    out.append((F, F.vals[0], bf[0]))
    V, bv, _ = W.varcoef_poisson5(50, seed=3)               # 2500 rows
    out.append((V, V.vals, bv))
    one = W.CSR(1, 1, np.array([0, 1], np.int32), np.array([0], np.int32), np.array([2.0]))
    out.append((one, one.vals, np.array([3.0])))
    P = W.poisson5(300)                                     # 90000 rows, many workgroups
    out.append((P, P.vals, W.rhs_uniform(P.n_rows, 4)))
    return out


def make_list(S, items, symmetric=True, jacobi_vals=None):
    rps = [dev(A.row_ptr.astype(np.int32)) for A, _, _ in items]
    cols = [dev(A.col.astype(np.int32)) for A, _, _ in items]
    return S.list_create(rps, cols, symmetric=symmetric)


def run(S, items, rtol, symmetric=True, max_iter=100000, fixed=False, jacobi=False, hist=None):
    h = make_list(S, items, symmetric=symmetric)
    opts = S.cg_opts(rtol=rtol, max_iter=max_iter, fixed=fixed, jacobi=jacobi, residual_history=hist)
    vals = [dev(v) for _, v, _ in items]
    b = [dev(bb) for _, _, bb in items]
    x, info = S.list_solve(h, vals, b, opts)
    gb, gv, binfo = S.list_solve_backward(h, vals, x, [xi.clone() for xi in x],
                                          S.cg_opts(rtol=rtol, max_iter=max_iter, fixed=fixed, jacobi=jacobi))
    return ([host(t) for t in x], [host(t) for t in gb], [host(t) for t in gv], S.read_info(info),
            S.read_info(binfo))


def check(items, out, rtol, max_iter=100000, fixed=False, jacobi=False):
    x, lam, gv, info, binfo = out
    tol_x, tol_adj = (1e-12, 1e-12) if fixed else (1e-9, 1e-8)
    for i, (A, v, b) in enumerate(items):
        f = O.cg(A, b, rtol=rtol, max_iter=max_iter, fixed=fixed, vals=v, jacobi=jacobi)
        assert info[i]["state"] == f["state"], (i, info[i], f["state"])
        assert iters_close(info[i]["iterations"], f["iterations"]), (i, info[i]["iterations"], f["iterations"])
        assert rel(x[i], f["x"]) <= tol_x, (i, rel(x[i], f["x"]))
        bw = O.solve_backward(A, x[i], x[i], symmetric=True, rtol=rtol, max_iter=max_iter, fixed=fixed, vals=v,
                              jacobi=jacobi)
        assert binfo[i]["state"] == bw["state"], i
        assert iters_close(binfo[i]["iterations"], bw["iterations"]), (i, binfo[i]["iterations"], bw["iterations"])
        assert rel(lam[i], bw["lam"]) <= tol_adj, (i, rel(lam[i], bw["lam"]))
        assert rel(gv[i], bw["gvals"]) <= tol_adj, (i, rel(gv[i], bw["gvals"]))


def test_list_mixed_items(S, schedule):
    items = items_mixed()
    out = run(S, items, rtol=1e-10)
    check(items, out, rtol=1e-10)
    assert len({i["iterations"] for i in out[3]}) == len(items)    # each item stops on its own


def test_list_transpose_path_is_the_symmetric_path(S):
    items = items_mixed()[:3]
    a = run(S, items, rtol=1e-10, symmetric=True)
    b = run(S, items, rtol=1e-10, symmetric=False)
    for k in range(3):
        for i in range(3):
            assert np.array_equal(a[k][i], b[k][i]), (k, i)


def test_list_jacobi(S):
    items = items_mixed()[1:3]
    out = run(S, items, rtol=1e-10, jacobi=True)
    check(items, out, rtol=1e-10, jacobi=True)


def test_list_fixed_iterations_and_histories(S):
    items = items_mixed()[:3]
    K = 8
    hist = torch.full((len(items), K + 1), float("nan"), dtype=torch.float64, device="cuda")
    out = run(S, items, rtol=0.0, max_iter=K, fixed=True, hist=hist)
    check(items, out, rtol=0.0, max_iter=K, fixed=True)
    hh = host(hist)
    for i, (A, v, b) in enumerate(items):
        f = O.cg(A, b, rtol=0.0, max_iter=K, fixed=True, vals=v, history=True)
        assert rel(hh[i], f["history"]) <= 1e-12, i


def test_list_matches_separate_solves(S):
    # the same items through sla_solve one by one: the same iterates to rounding
    items = items_mixed()[:3]
    K = 10
    lx = run(S, items, rtol=0.0, max_iter=K, fixed=True)[0]
    for i, (A, v, b) in enumerate(items):
        h = S.csr_create(dev(A.row_ptr.astype(np.int32)), dev(A.col.astype(np.int32)), symmetric=True)
        x, _ = S.solve(h, dev(v), dev(b), S.cg_opts(rtol=0.0, max_iter=K, fixed=True))
        assert rel(lx[i], host(x)) <= 1e-13, i


def test_list_mixed_outcomes(S):
    base = items_mixed()[:3]
    A0, v0, b0 = base[0]
    A1, v1, b1 = base[1]
    A2, v2, b2 = base[2]
    v_nan = v2.copy()
    v_nan[5] = np.nan
    items = [(A0, v0, np.zeros_like(b0)),     # b = 0: converged, 0 iterations
             (A1, -v1, b1),                   # -A: not SPD at the first step
             (A2, v_nan, b2),                 # NaN
             (A0, v0, b0)]                    # a normal solve beside them
    h = make_list(S, items)
    x, info = S.list_solve(h, [dev(v) for _, v, _ in items], [dev(b) for _, _, b in items],
                           S.cg_opts(rtol=1e-10))
    inf = S.read_info(info)
    assert [i["state"] for i in inf] == [O.CONVERGED, O.NOT_SPD, O.NAN, O.CONVERGED]
    assert inf[0]["iterations"] == 0 and not np.any(host(x[0]))
    f = O.cg(A0, b0, rtol=1e-10, vals=v0)
    assert iters_close(inf[3]["iterations"], f["iterations"]) and rel(host(x[3]), f["x"]) <= 1e-9


def test_list_rejects_a_bad_item(S):
    A = W.poisson5(10)
    bad = A.col.copy()
    bad[-1] = A.n_rows            # a column past its own item's rows
    with pytest.raises(S.SlaError):
        S.list_create([dev(A.row_ptr), dev(A.row_ptr)], [dev(A.col), dev(bad)], symmetric=True)


def test_list_autograd(S):
    items = items_mixed()[:4]
    T = S.SparseTensorList([dev(A.row_ptr.astype(np.int32)) for A, _, _ in items],
                           [dev(A.col) for A, _, _ in items],
                           [dev(v).requires_grad_(True) for _, v, _ in items], symmetric=True)
    bs = [dev(b).requires_grad_(True) for _, _, b in items]
    xs = T.solve(bs, rtol=1e-12)
    sum(0.5 * (x * x).sum() for x in xs).backward()
    for i, (A, v, b) in enumerate(items):
        f = O.cg(A, b, rtol=1e-12, vals=v)
        bw = O.solve_backward(A, f["x"], f["x"], symmetric=True, rtol=1e-12, vals=v)
        assert rel(host(xs[i]), f["x"]) <= 1e-9
        assert rel(host(bs[i].grad), bw["lam"]) <= 1e-8
        assert rel(host(T.vals[i].grad), bw["gvals"]) <= 1e-8
