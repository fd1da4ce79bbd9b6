"""GPU parity of the diagonal-layout banded CG SpMV (k_cg_spmv_dia), through the C ABI.

A banded pattern whose stored offsets c - i take at most 16 distinct values gets a
diagonal layout at create: one value per diagonal and row (copied from the CSR values
once per solve) and a per-row mask of the diagonals the row stores.  Each row sum is
the CSR row sum in the same (ascending column) order, and the inner products are
summed over the same lanes, so every result must equal the staged banded kernel's --
the same handle built with SLA_DIA=0 -- to the bit, and the oracle's to the usual bars.  Cases: the 5-point grid (5 diagonals, 8-bit masks, the
5-slot kernel), a 7-diagonal pattern (8-slot kernel), the 9-point grid (16-slot kernel,
16-bit masks), a grid with symmetric pairs of entries removed (rows that skip
diagonals), a last line cut short, a batch, Jacobi PCG, fixed iterations with the
residual history, a 19-diagonal pattern (no layout: the staged kernel), and a grid at
the default minimum stride with several blocks per workgroup.  Line strides of 8
(mod 16) take windows shifted onto 128-byte boundaries by default: those are held to the
oracle, and to the unshifted layout over fixed iterations; strides 504 and 280 put the
shifted last window at its widest and near its narrowest.
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
    return monkeypatch


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def from_triplets(n, rows, cols, vals):
    o = np.lexsort((cols, rows))
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows[o] + 1, 1)
    return W.CSR(n, n, np.cumsum(rp).astype(np.int32), cols[o].astype(np.int32), vals[o])


def offsets_matrix(n, offsets, diag):
    """Symmetric banded matrix with entries at c = i + d for every d in offsets (those
    in range), -1 off the diagonal and `diag` on it (diagonally dominant: SPD)."""
    rows, cols, vals = [], [], []
    i = np.arange(n)
    for d in offsets:
        ok = (i + d >= 0) & (i + d < n)
        rows.append(i[ok])
        cols.append(i[ok] + d)
        vals.append(np.full(int(ok.sum()), diag if d == 0 else -1.0))
    return from_triplets(n, *map(np.concatenate, (rows, cols, vals)))


def nine_point(nx, ny):
    rows, cols, vals = [], [], []
    a, c = np.divmod(np.arange(nx * ny), nx)
    for da in (-1, 0, 1):
        for dc in (-1, 0, 1):
            ok = (a + da >= 0) & (a + da < ny) & (c + dc >= 0) & (c + dc < nx)
            i = np.nonzero(ok)[0]
            rows.append(i)
            cols.append((a[i] + da) * nx + c[i] + dc)
            vals.append(np.full(i.size, 8.0 if (da, dc) == (0, 0) else -1.0))
    return from_triplets(nx * ny, *map(np.concatenate, (rows, cols, vals)))


def drop_pairs(A, frac, seed):
    """A with a random set of symmetric off-diagonal pairs removed (still SPD: the
    diagonal stays, so every row remains diagonally dominant)."""
    rng = np.random.default_rng(seed)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))
    up = np.nonzero(A.col > rows)[0]
    kill = up[rng.random(up.size) < frac]
    dead = set(zip(rows[kill].tolist(), A.col[kill].tolist()))
    dead |= {(c, r) for r, c in dead}
    keep = np.array([(r, c) not in dead for r, c in zip(rows.tolist(), A.col.tolist())])
    return from_triplets(A.n_rows, rows[keep], A.col[keep], A.vals[keep])


def leading(A, m):
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr.astype(np.int64)))
    keep = (rows < m) & (A.col < m)
    return from_triplets(m, rows[keep], A.col[keep], A.vals[keep])


def run(S, h, vals, b, opts, jac=False):
    x, info = S.solve(h, vals, b, opts)
    gb, gv, binfo = S.solve_backward(h, vals, x, x.clone(), opts)
    return [host(t) for t in (x, gb, gv)], S.read_info(info), S.read_info(binfo)


def both(S, A, b, opts, monkeypatch, vals=None):
    """The same solve + adjoint with the diagonal layout's windows unshifted
    (SLA_DIA_ALIGN=0), with the staged banded kernel (SLA_DIA=0) and with the default
    layout, whose windows on every other line start 8 rows early when the line stride is
    8 (mod 16) so that they sit on 128-byte boundaries.  All handles have the same band.
    The unshifted layout sums every row in the staged kernel's order and in the same
    workgroup, so it must match it to the bit; the shifted one sums the same rows in the
    same order, but some in another workgroup (the grouping of p^T q's partials)."""
    vals = A.vals if vals is None else vals
    rp, col = dev(A.row_ptr.astype(np.int32)), dev(A.col.astype(np.int32))
    ha = S.csr_create(rp, col, symmetric=True)
    monkeypatch.setenv("SLA_DIA_ALIGN", "0")
    hd = S.csr_create(rp, col, symmetric=True)
    monkeypatch.delenv("SLA_DIA_ALIGN")
    monkeypatch.setenv("SLA_DIA", "0")
    hs = S.csr_create(rp, col, symmetric=True)
    monkeypatch.delenv("SLA_DIA")
    ad, as_ = S.csr_analysis(hd), S.csr_analysis(hs)
    assert ad["band_stride"] == as_["band_stride"] > 0 and as_["diagonals"] == 0
    assert S.csr_analysis(ha)["diagonals"] == ad["diagonals"]
    dv, db = dev(vals), dev(b)
    return ad, run(S, hd, dv, db, opts), run(S, hs, dv, db, opts), run(S, ha, dv, db, opts)


def assert_bit_identical(r_dia, r_staged):
    (v1, i1, b1), (v2, i2, b2) = r_dia, r_staged
    for a, c in zip(v1, v2):
        assert np.array_equal(a, c)
    assert i1 == i2 and b1 == b2


def check_oracle(A, b, res, rtol, vals=None):
    (x, lam, gv), info, binfo = res
    f = O.cg(A, b, rtol=rtol, vals=vals)
    bw = O.solve_backward(A, x, x, symmetric=True, rtol=rtol, vals=vals)
    assert abs(info[0]["iterations"] - f["iterations"]) <= math.floor(0.02 * f["iterations"])
    assert rel(x, f["x"]) <= 1e-9 and rel(lam, bw["lam"]) <= 1e-8 and rel(gv, bw["gvals"]) <= 1e-8


@pytest.mark.parametrize("case", ["poisson520", "seven", "nine", "dropped", "cut",
                                  "poisson600", "seven600", "nine599", "dropped599", "cut600",
                                  "poisson504", "poisson280"])
def test_dia_equals_staged_band_and_oracle(S, band_env, case):
    if case == "poisson520":
        A, nd = W.poisson5(520), 5
    elif case == "seven":
        A, nd = offsets_matrix(300 * 40, [-300, -2, -1, 0, 1, 2, 300], 6.5), 7
    elif case == "nine":
        A, nd = nine_point(300, 12), 9
    elif case == "dropped":
        A, nd = drop_pairs(nine_point(300, 10), 0.3, seed=3), 9
    elif case == "cut":
        A, nd = leading(W.poisson5(300), 300 * 9 - 37), 5
    elif case == "poisson600":
        A, nd = W.poisson5(600), 5
    elif case == "seven600":
        A, nd = offsets_matrix(600 * 30, [-600, -2, -1, 0, 1, 2, 600], 6.5), 7
    elif case == "nine599":      # stride 600
        A, nd = nine_point(599, 12), 9
    elif case == "dropped599":
        A, nd = drop_pairs(nine_point(599, 10), 0.3, seed=4), 9
    elif case == "cut600":       # a last line cut short, n even
        A, nd = leading(W.poisson5(600), 600 * 9 - 38), 5
    elif case == "poisson504":   # 504 = 248 (mod 256): shifted last windows are exactly 256 rows
        A, nd = leading(W.poisson5(504), 504 * 40), 5
    else:                        # 280 = 24 (mod 256): last windows of 24 and 32 rows
        A, nd = leading(W.poisson5(280), 280 * 40), 5
    b = W.rhs_normal(A.n_rows, 11)
    ad, rd, rs, ra = both(S, A, b, S.cg_opts(rtol=1e-10), band_env)
    assert ad["diagonals"] == nd
    assert_bit_identical(rd, rs)
    check_oracle(A, b, rd, 1e-10)
    check_oracle(A, b, ra, 1e-10)


def test_dia_fixed_iterations_history(S, band_env):
    A = W.poisson5(520)
    b = W.rhs_normal(A.n_rows, 4)
    K = 60
    rp, col = dev(A.row_ptr), dev(A.col)
    h = S.csr_create(rp, col, symmetric=True)
    assert S.csr_analysis(h)["diagonals"] == 5
    hist = torch.full((K + 1,), float("nan"), dtype=torch.float64, device="cuda")
    x, info = S.solve(h, dev(A.vals), dev(b), S.cg_opts(rtol=0.0, max_iter=K, fixed=True, residual_history=hist))
    f = O.cg(A, b, rtol=0.0, max_iter=K, fixed=True, history=True)
    assert S.read_info(info)[0]["iterations"] == K
    assert rel(host(hist), f["history"]) <= 1e-12 and rel(host(x), f["x"]) <= 1e-12


def test_dia_batch_and_jacobi(S, band_env):
    A = W.poisson5(300)
    B = 3
    vals = np.stack([A.vals * (1.0 + 0.5 * s) for s in range(B)])
    b = np.stack([W.rhs_normal(A.n_rows, 20 + s) for s in range(B)])
    ad, rd, rs, ra = both(S, A, b, S.cg_opts(rtol=1e-10), band_env, vals=vals)
    assert ad["diagonals"] == 5
    assert_bit_identical(rd, rs)
    for s in range(B):
        f = O.cg(A, b[s], rtol=1e-10, vals=vals[s])
        assert rel(rd[0][0][s], f["x"]) <= 1e-9 and rel(ra[0][0][s], f["x"]) <= 1e-9
    # Jacobi on a variable-coefficient grid (its diagonal is not constant)
    V, bv, _ = W.varcoef_poisson5(300, seed=5)
    ad, rd, rs, ra = both(S, V, bv, S.cg_opts(rtol=1e-10, jacobi=True), band_env)
    assert ad["diagonals"] == 5
    assert_bit_identical(rd, rs)
    f = O.cg(V, bv, rtol=1e-10, jacobi=True)
    for r in (rd, ra):
        assert abs(r[1][0]["iterations"] - f["iterations"]) <= math.floor(0.02 * f["iterations"])
        assert rel(r[0][0], f["x"]) <= 1e-9


def test_dia_too_many_diagonals_keeps_the_staged_kernel(S, band_env):
    # 21 distinct offsets but at most 11 entries per row: the first half of the rows
    # couples among themselves at offsets 0, +-1..3, +-300, the second half at 0,
    # +-4..8, +-299 (each pair stays within its half, so the matrix is symmetric)
    n = 300 * 30
    h2 = n // 2
    rows, cols, vals = [], [], []
    i = np.arange(n)
    for lo, hi, offs in ((0, h2, [0, 1, 2, 3, 300]), (h2, n, [0, 4, 5, 6, 7, 8, 299])):
        for d in offs:
            for sgn in ((1,) if d == 0 else (1, -1)):
                c = i + sgn * d
                ok = (i >= lo) & (i < hi) & (c >= lo) & (c < hi)
                rows.append(i[ok])
                cols.append(c[ok])
                vals.append(np.full(int(ok.sum()), 20.0 if d == 0 else -1.0))
    A = from_triplets(n, *map(np.concatenate, (rows, cols, vals)))
    h = S.csr_create(dev(A.row_ptr), dev(A.col), symmetric=True)
    an = S.csr_analysis(h)
    assert an["band_stride"] == 300 and an["diagonals"] == 0
    b = W.rhs_normal(A.n_rows, 1)
    x, info = S.solve(h, dev(A.vals), dev(b), S.cg_opts(rtol=1e-10))
    f = O.cg(A, b, rtol=1e-10)
    assert rel(host(x), f["x"]) <= 1e-9


def test_dia_several_blocks_per_workgroup(S, monkeypatch):
    # 3000 x 3000 at the default minimum stride: the diagonal layout, bit for bit the
    # staged kernel over 12 fixed iterations, and the oracle's
    A = W.poisson5(3000)
    b = W.rhs_normal(A.n_rows, 8)
    K = 12
    ad, rd, rs, ra = both(S, A, b, S.cg_opts(rtol=0.0, max_iter=K, fixed=True), monkeypatch)
    assert ad["diagonals"] == 5 and ad["band_stride"] == 3000
    assert_bit_identical(rd, rs)
    f = O.cg(A, b, rtol=0.0, max_iter=K, fixed=True)
    assert rel(rd[0][0], f["x"]) <= 1e-12
    # the shifted windows (3000 = 8 mod 16): the same iterates to rounding
    for a_, c_ in zip(ra[0], rd[0]):
        assert rel(a_, c_) <= 1e-12
    assert rel(ra[0][0], f["x"]) <= 1e-12


def test_dia_aligned_windows_batch(S, band_env):
    # a batch of three systems at stride 520 (8 mod 16: shifted windows) against the
    # oracle, and the unshifted layout bit for bit against the staged kernel
    A = leading(W.poisson5(520), 520 * 60)
    B = 3
    vals = np.stack([A.vals * (1.0 + 0.25 * s) for s in range(B)])
    b = np.stack([W.rhs_normal(A.n_rows, 40 + s) for s in range(B)])
    ad, rd, rs, ra = both(S, A, b, S.cg_opts(rtol=1e-10), band_env, vals=vals)
    assert ad["diagonals"] == 5 and ad["band_stride"] == 520
    assert_bit_identical(rd, rs)
    for s in range(B):
        f = O.cg(A, b[s], rtol=1e-10, vals=vals[s])
        bw = O.solve_backward(A, ra[0][0][s], ra[0][0][s], symmetric=True, rtol=1e-10, vals=vals[s])
        assert abs(ra[1][s]["iterations"] - f["iterations"]) <= math.floor(0.02 * f["iterations"])
        assert rel(ra[0][0][s], f["x"]) <= 1e-9
        assert rel(ra[0][1][s], bw["lam"]) <= 1e-8 and rel(ra[0][2][s], bw["gvals"]) <= 1e-8
