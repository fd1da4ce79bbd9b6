"""GPU tests of the 16-bit column offsets (sla_csr_create, "Column offsets"), through
the C ABI.

The plain CG and BiCGStab SpMV (and the Lanczos product) read 16-bit offsets c - row0
(row0 the first row of the entry's 256-row tile) in place of the 32-bit columns when
every stored entry has |c - i| <= 32512.  The offsets change only how the columns are
read, not the sums: every result must be bit for bit that of the same handle created
with SLA_COL16=0.  The patterns include the extreme offsets +32767 and -32512 (entries
at |c - i| = 32512 in the last and the first row of a tile), the first span past the
limit (no offsets), the split schedule, the transposed adjoint of BiCGStab, a
SparseTensorList and Lanczos.  Against the oracle the solves keep the single-system
bars (iterations within 2 %, x within 1e-9, lambda and dL/dvals within 1e-8).
"""
import math

import numpy as np
import pytest
import scipy.sparse as sp

import oracle as O
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SPAN = 32512          # the largest |c - i| that still takes offsets


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


def csr_of(M):
    M = sp.csr_matrix(M)
    M.sort_indices()
    return W.CSR(M.shape[0], M.shape[1], M.indptr.astype(np.int32), M.indices.astype(np.int32),
                 M.data.astype(np.float64))


def far_pairs(n, span):
    """An SPD matrix: 1D Laplacian (2, -1) plus 0.5 I, and symmetric couplings -0.25 at
    distance `span` from row 255 (last row of tile 0: offset 255 + span) and from row
    span + 256 (first row of its tile, coupled to row 256: offset -span)."""
    M = sp.diags([-np.ones(n - 1), 2.5 * np.ones(n), -np.ones(n - 1)], [-1, 0, 1], format="lil")
    for i in (255, 256):
        M[i, i + span] = -0.25
        M[i + span, i] = -0.25
    return csr_of(M.tocsr())


def handle(S, A, monkeypatch, c16, symmetric=True):
    monkeypatch.setenv("SLA_COL16", "1" if c16 else "0")
    h = S.csr_create(dev(A.row_ptr), dev(A.col), symmetric=symmetric)
    monkeypatch.delenv("SLA_COL16")
    return h


def solve_both(S, h, A, b, opts):
    x, info = S.solve(h, dev(A.vals), dev(b), opts)
    gb, gv, binfo = S.solve_backward(h, dev(A.vals), x, x.clone(), opts)
    return [host(x), host(gb), host(gv)], S.read_info(info)[0], S.read_info(binfo)[0]


def same(S, A, b, monkeypatch, opts, symmetric=True, expect_bits=16):
    ha = handle(S, A, monkeypatch, True, symmetric)
    hb = handle(S, A, monkeypatch, False, symmetric)
    assert S.csr_analysis(ha)["col_bits"] == expect_bits
    assert S.csr_analysis(hb)["col_bits"] == 32
    ra, ia, ba = solve_both(S, ha, A, b, opts)
    rb, ib, bb = solve_both(S, hb, A, b, opts)
    for u, v in zip(ra, rb):
        assert np.array_equal(u, v)
    assert ia == ib and ba == bb
    return ra, ia, ba


def test_offsets_at_the_limit(S, monkeypatch):
    n = 2 * SPAN + 600
    A = far_pairs(n, SPAN)
    b = W.rhs_normal(n, 1)
    (x, lam, gv), info, binfo = same(S, A, b, monkeypatch, S.cg_opts(rtol=1e-10))
    f = O.cg(A, b, rtol=1e-10)
    assert info["state"] == f["state"] == O.CONVERGED
    assert abs(info["iterations"] - f["iterations"]) <= math.floor(0.02 * f["iterations"])
    assert rel(x, f["x"]) <= 1e-9
    bw = O.solve_backward(A, x, x, symmetric=True, rtol=1e-10)
    assert rel(lam, bw["lam"]) <= 1e-8 and rel(gv, bw["gvals"]) <= 1e-8


def test_no_offsets_past_the_limit(S, monkeypatch):
    A = far_pairs(2 * SPAN + 600, SPAN + 1)
    h = handle(S, A, monkeypatch, True)
    assert S.csr_analysis(h)["col_bits"] == 32


@pytest.mark.parametrize("schedule", ["fused", "split"])
def test_cg_schedules_bit_identical(S, monkeypatch, schedule):
    monkeypatch.setenv("SLA_CG_SCHEDULE", schedule)
    A = W.poisson5(300)                  # 90000 rows, a ragged last tile
    same(S, A, W.rhs_normal(A.n_rows, 2), monkeypatch, S.cg_opts(rtol=1e-9))
    F, bf = W.fem_p1_batched(nv=60, B=1, seed=4)      # scattered vertex ids
    F1 = W.CSR(F.n_rows, F.n_cols, F.row_ptr, F.col, F.vals[0])
    same(S, F1, bf[0], monkeypatch, S.cg_opts(rtol=1e-9))


def test_bicgstab_and_transposed_adjoint_bit_identical(S, monkeypatch):
    A = W.convdiff5(200, wind=100.0, shift=1.0)
    b = W.rhs_normal(A.n_rows, 3)
    opts = S.cg_opts(rtol=1e-9, method="bicgstab")
    (x, lam, gv), info, binfo = same(S, A, b, monkeypatch, opts, symmetric=False)
    f = O.cg(A, b, rtol=1e-9, method="bicgstab")
    assert rel(x, f["x"]) <= 1e-9


def test_list_bit_identical(S, monkeypatch):
    items = [W.poisson5(40), W.poisson5(70), far_pairs(2 * SPAN + 600, SPAN)]
    bs = [W.rhs_normal(A.n_rows, 5 + i) for i, A in enumerate(items)]
    out = []
    for c16 in (True, False):
        monkeypatch.setenv("SLA_COL16", "1" if c16 else "0")
        h = S.list_create([dev(A.row_ptr) for A in items], [dev(A.col) for A in items], symmetric=True)
        monkeypatch.delenv("SLA_COL16")
        assert S.list_col_bits(h) == (16 if c16 else 32)
        x, info = S.list_solve(h, [dev(A.vals) for A in items], [dev(b) for b in bs], S.cg_opts(rtol=1e-10))
        out.append(([host(t) for t in x], S.read_info(info)))
    for u, v in zip(out[0][0], out[1][0]):
        assert np.array_equal(u, v)
    assert out[0][1] == out[1][1]


def test_lanczos_bit_identical(S, monkeypatch):
    A, _, _ = W.varcoef_poisson5(120, seed=2)
    v0 = dev(W.rhs_normal(A.n_rows, 4))
    res = []
    for c16 in (True, False):
        h = handle(S, A, monkeypatch, c16)
        ev, U, info = S.eigsh(h, dev(A.vals), 4, v0, which="largest", tol=1e-10)
        res.append((host(ev), host(U), info))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    assert res[0][2] == res[1][2]


def laplacian_rect(nx, ny):
    """5-point Laplacian (4, -1) on an nx x ny grid in natural order (line stride nx)."""
    Tx = sp.diags([-np.ones(nx - 1), 2 * np.ones(nx), -np.ones(nx - 1)], [-1, 0, 1])
    Ty = sp.diags([-np.ones(ny - 1), 2 * np.ones(ny), -np.ones(ny - 1)], [-1, 0, 1])
    return csr_of(sp.kron(sp.eye(ny), Tx) + sp.kron(Ty, sp.eye(nx)))


@pytest.mark.parametrize("nx,ny,fixed", [(300, 300, False), (SPAN, 4, True)])
def test_banded_bit_identical(S, monkeypatch, nx, ny, fixed):
    # the line-walking SpMV reads offsets from each window's first row: strips of 256
    # and 44 positions (stride 300), and the largest stride that takes offsets (the
    # last row of a window reaching S + 255 = 32767)
    monkeypatch.setenv("SLA_BAND_MIN_STRIDE", "272")
    A = laplacian_rect(nx, ny)
    b = W.rhs_normal(A.n_rows, 6)
    opts = S.cg_opts(rtol=0.0, max_iter=40, fixed=True) if fixed else S.cg_opts(rtol=1e-10)
    ha = handle(S, A, monkeypatch, True)
    assert S.csr_analysis(ha)["band_stride"] == nx
    (x, lam, gv), info, _ = same(S, A, b, monkeypatch, opts)
    if fixed:
        f = O.cg(A, b, rtol=0.0, max_iter=40, fixed=True)
        assert info["iterations"] == 40 and rel(x, f["x"]) <= 1e-12
    else:
        f = O.cg(A, b, rtol=1e-10)
        assert abs(info["iterations"] - f["iterations"]) <= math.floor(0.02 * f["iterations"])
        assert rel(x, f["x"]) <= 1e-9
