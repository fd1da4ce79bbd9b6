"""GPU parity of the line-walking SpMV for banded patterns, through the C ABI.

The band analysis at csr_create picks this SpMV for square patterns whose entries all
lie within 8 of the diagonal or within 8 below the largest distance S (grid stencils in
natural order), once S reaches the minimum stride (2048 by default).  These tests lower
the minimum through SLA_BAND_MIN_STRIDE so that grids of a few hundred lines take it,
and hold it to the same bars as the plain SpMV against the oracle: iterations within
2 %, x within 1e-9, lambda and dL/dvals within 1e-8 (1e-12 over fixed iterations).
Cases: strips of 256 positions with a ragged last strip (N = 520: 256 + 256 + 8), a
last line cut short (n not a multiple of S) that also leaves a block of one line, a
9-point stencil (S = N + 1, 9 entries per row, the widest LDS variant), a batch of
systems sharing the pattern, and a grid (N = 3000) with more blocks of lines than
workgroups, so that workgroups take several blocks one after the other.
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


@pytest.fixture
def band_env(monkeypatch):
    monkeypatch.setenv("SLA_BAND_MIN_STRIDE", "1")


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


def grid_stencil(nx, ny, nine=False):
    """Dirichlet Laplacian on an nx x ny grid in natural order (unknown (a, c) -> a nx + c):
    5-point (4, -1) or 9-point (8, -1) stencil.  Both are SPD."""
    offs = [(da, dc) for da in (-1, 0, 1) for dc in (-1, 0, 1)
            if (da, dc) != (0, 0) and (nine or da == 0 or dc == 0)]
    offs = sorted(offs + [(0, 0)])          # lexicographic = ascending column
    diag = 8.0 if nine else 4.0
    rows, cols, vals = [], [], []
    a, c = np.divmod(np.arange(nx * ny), nx)
    for da, dc in offs:
        ok = (a + da >= 0) & (a + da < ny) & (c + dc >= 0) & (c + dc < nx)
        i = np.nonzero(ok)[0]
        rows.append(i)
        cols.append((a[i] + da) * nx + c[i] + dc)
        vals.append(np.full(i.size, diag if (da, dc) == (0, 0) else -1.0))
    rows, cols, vals = map(np.concatenate, (rows, cols, vals))
    order = np.lexsort((cols, rows))
    rows, cols, vals = rows[order], cols[order], vals[order]
    n = nx * ny
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    rp = np.cumsum(rp)
    return W.CSR(n, n, rp.astype(np.int32), cols.astype(np.int32), vals)


def leading(A, m):
    """Leading m x m block of A (SPD when A is)."""
    keep_r = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64))) < m
    keep = keep_r & (A.col < m)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))[keep]
    rp = np.zeros(m + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    return W.CSR(m, m, np.cumsum(rp).astype(np.int32), A.col[keep].astype(np.int32), A.vals[keep])


def run_pair(S, A, b, rtol, vals=None, max_iter=100000, fixed=False):
    """GPU solve + adjoint (L = 0.5 |x|^2 per system) and the oracle's."""
    vals = A.vals.reshape(1, -1) if vals is None else vals
    B = vals.shape[0]
    b = b.reshape(B, A.n_rows)
    h = handle(S, A)
    an = S.csr_analysis(h)
    opts = S.cg_opts(rtol=rtol, max_iter=max_iter, fixed=fixed)
    dv = dev(vals)
    x, info = S.solve(h, dv, dev(b), opts)
    gb, gv, binfo = S.solve_backward(h, dv, x, x.clone(), opts)
    xg, lam, gvals = host(x), host(gb), host(gv)
    info, binfo = S.read_info(info), S.read_info(binfo)
    for s in range(B):
        f = O.cg(A, b[s], rtol=rtol, max_iter=max_iter, fixed=fixed, vals=vals[s])
        bw = O.solve_backward(A, xg[s], xg[s], symmetric=True, rtol=rtol, max_iter=max_iter, fixed=fixed,
                              vals=vals[s])
        tol_x, tol_adj = (1e-12, 1e-12) if fixed else (1e-9, 1e-8)
        assert info[s]["state"] == f["state"], (s, info[s], f["state"])
        assert iters_close(info[s]["iterations"], f["iterations"]), (s, info[s]["iterations"], f["iterations"])
        assert rel(xg[s], f["x"]) <= tol_x, (s, rel(xg[s], f["x"]))
        assert binfo[s]["state"] == bw["state"]
        assert iters_close(binfo[s]["iterations"], bw["iterations"]), (s, binfo[s]["iterations"],
                                                                       bw["iterations"])
        assert rel(lam[s], bw["lam"]) <= tol_adj, (s, rel(lam[s], bw["lam"]))
        assert rel(gvals[s], bw["gvals"]) <= tol_adj, (s, rel(gvals[s], bw["gvals"]))
    return an


def test_band_analysis(S, monkeypatch):
    A = W.poisson5(300)
    assert S.csr_analysis(handle(S, A))["band_stride"] == 0        # below the default 2048
    monkeypatch.setenv("SLA_BAND_MIN_STRIDE", "1")
    an = S.csr_analysis(handle(S, A))
    assert an["band_stride"] == 300 and an["row_max"] == 5 and an["spmv_cap"] == 1280
    an = S.csr_analysis(handle(S, grid_stencil(300, 6, nine=True)))
    assert an["band_stride"] == 301 and an["row_max"] == 9 and an["spmv_cap"] == 4096
    assert S.csr_analysis(handle(S, W.poisson5(200)))["band_stride"] == 0   # S < 272: segments overlap
    fem, _ = W.fem_p1_batched(nv=30, B=1, seed=2)
    assert S.csr_analysis(handle(S, fem))["band_stride"] == 0       # permuted mesh: no band
    # one symmetric pair of entries at distance 150 breaks the band
    D = W.poisson5(300)
    rows = np.repeat(np.arange(D.n_rows), np.diff(D.row_ptr.astype(np.int64)))
    extra_r, extra_c = np.array([1000, 1150]), np.array([1150, 1000])
    r2 = np.concatenate([rows, extra_r])
    c2 = np.concatenate([D.col, extra_c])
    o = np.lexsort((c2, r2))
    rp = np.zeros(D.n_rows + 1, np.int64)
    np.add.at(rp, r2[o] + 1, 1)
    E = W.CSR(D.n_rows, D.n_cols, np.cumsum(rp).astype(np.int32), c2[o].astype(np.int32),
              np.concatenate([D.vals, [-0.5, -0.5]])[o])
    assert S.csr_analysis(handle(S, E))["band_stride"] == 0


@pytest.mark.parametrize("N", [300, 520])
def test_band_cg_poisson(S, band_env, N):
    A = W.poisson5(N)
    an = run_pair(S, A, W.rhs_normal(A.n_rows, N), rtol=1e-10)
    assert an["band_stride"] == N


def test_band_fixed_iterations(S, band_env):
    A = W.poisson5(520)
    an = run_pair(S, A, W.rhs_normal(A.n_rows, 4), rtol=0.0, max_iter=120, fixed=True)
    assert an["band_stride"] == 520


def test_band_last_line_cut_short(S, band_env):
    A = leading(grid_stencil(300, 9), 300 * 9 - 37)
    an = run_pair(S, A, W.rhs_uniform(A.n_rows, 5), rtol=1e-10)
    assert an["band_stride"] == 300


def test_band_nine_point(S, band_env):
    A = grid_stencil(300, 12, nine=True)
    an = run_pair(S, A, W.rhs_normal(A.n_rows, 6), rtol=1e-10)
    assert an["band_stride"] == 301 and an["spmv_cap"] == 4096


def test_band_batched_shared_pattern(S, band_env):
    A = W.poisson5(300)
    B = 3
    vals = np.stack([A.vals * (1.0 + 0.5 * s) for s in range(B)])
    b = np.stack([W.rhs_normal(A.n_rows, 10 + s) for s in range(B)])
    an = run_pair(S, A, b, rtol=1e-10, vals=vals)
    assert an["band_stride"] == 300


def test_band_several_blocks_per_workgroup(S):
    # 3000 x 3000 (S = 3000 >= the default minimum stride): 12 strips x 94 blocks of 32
    # lines, more than the resident workgroups; 12 fixed iterations against the oracle.
    A = W.poisson5(3000)
    b = W.rhs_normal(A.n_rows, 8)
    h = handle(S, A)
    assert S.csr_analysis(h)["band_stride"] == 3000
    K = 12
    hist = torch.full((K + 1,), float("nan"), dtype=torch.float64, device="cuda")
    x, info = S.solve(h, dev(A.vals), dev(b), S.cg_opts(rtol=0.0, max_iter=K, fixed=True,
                                                          residual_history=hist))
    f = O.cg(A, b, rtol=0.0, max_iter=K, fixed=True, history=True)
    assert S.read_info(info)[0]["iterations"] == K
    assert rel(host(hist), f["history"]) <= 1e-12
    assert rel(host(x), f["x"]) <= 1e-12
