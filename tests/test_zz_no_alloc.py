"""sla_solve_noalloc, the allocation-free variant of sla_solve (its workspace in the
library's static device scratch), through the C ABI: its results equal sla_solve's on
the same inputs, bit for bit (the same kernels on the same data), on two calls in a
row, the second with a smaller problem (the scratch keeps the first call's contents,
which the second must not read); it allocates nothing (the torch allocator registered
with the library sees no call); and a problem beyond the scratch is refused before any
launch."""
import gc

import numpy as np
import pytest

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


def both(S, h, vals, b, opts):
    B = vals.shape[0] if vals.dim() == 2 else 1
    x_ref, info_ref = S.solve(h, vals, b, opts)
    x = torch.full_like(b, float("nan"))
    info = S.info_buffer(B, b.device)
    S.solve_noalloc(h, vals, b, opts, x, info)
    torch.cuda.synchronize()
    return (x_ref.cpu().numpy(), S.read_info(info_ref)), (x.cpu().numpy(), S.read_info(info))


def check_equal(ref, out):
    (xr, ir), (xo, io) = ref, out
    assert np.array_equal(xr, xo)
    assert [(i["iterations"], i["state"], i["res_norm"]) for i in ir] == \
        [(i["iterations"], i["state"], i["res_norm"]) for i in io]


def test_noalloc_matches_solve_on_two_calls_in_a_row(S):
    from differentiable_sparse_linear_spmv_amd import _lib as L
    lib = L.load()
    calls = {"n": 0}

    def _alloc(size, stream, ctx):
        calls["n"] += 1
        return torch.cuda.caching_allocator_alloc(int(size))

    def _free(ptr, stream, ctx):
        torch.cuda.caching_allocator_delete(ptr)

    # first call: a batch of 3 varcoef systems (ragged last tile), Jacobi CG
    A1, b1, _ = W.varcoef_poisson5(150, seed=4)
    vals1 = dev(np.stack([A1.vals, 2.0 * A1.vals, A1.vals + 0.5 * (A1.vals > 0)]))
    bb1 = dev(np.stack([b1, W.rhs_normal(A1.n_rows, 7), b1[::-1]]))
    h1 = S.csr_create(dev(A1.row_ptr), dev(A1.col), symmetric=True)
    o1 = S.cg_opts(rtol=1e-10, jacobi=True)
    # second call: a smaller single system, plain CG, on another handle
    A2 = W.poisson5(60)
    h2 = S.csr_create(dev(A2.row_ptr), dev(A2.col), symmetric=True)
    vals2, bb2 = dev(A2.vals), dev(W.rhs_normal(A2.n_rows, 9))
    o2 = S.cg_opts(rtol=1e-10)
    # sla_solve's reference results first (these allocate the handles' workspaces)
    ref1 = both(S, h1, vals1, bb1, o1)[0]
    ref2 = both(S, h2, vals2, bb2, o2)[0]
    cbs = (L.ALLOC_FN(_alloc), L.FREE_FN(_free))
    assert lib.sla_set_allocator(cbs[0], cbs[1], None) == 0
    try:
        B1 = 3
        x1 = torch.full_like(bb1, float("nan"))
        i1 = S.info_buffer(B1, bb1.device)
        S.solve_noalloc(h1, vals1, bb1, o1, x1, i1)
        x2 = torch.full_like(bb2, float("nan"))
        i2 = S.info_buffer(1, bb2.device)
        S.solve_noalloc(h2, vals2, bb2, o2, x2, i2)
        torch.cuda.synchronize()
        assert calls["n"] == 0, calls
        check_equal(ref1, (x1.cpu().numpy(), S.read_info(i1)))
        check_equal(ref2, (x2.cpu().numpy(), S.read_info(i2)))
        assert all(i["state"] == 0 for i in S.read_info(i1) + S.read_info(i2))
    finally:
        assert lib.sla_set_allocator(L.ALLOC_FN(), L.FREE_FN(), None) == 0


def test_noalloc_bicgstab_and_banded(S, monkeypatch):
    # BiCGStab on a nonsymmetric system, and CG on a banded handle (whose plain-kernel
    # column offsets are not built: the banded SpMV reads its own)
    A = W.convdiff5(120, wind=20.0, shift=0.5)
    h = S.csr_create(dev(A.row_ptr), dev(A.col), symmetric=False)
    vals, b = dev(A.vals), dev(W.rhs_normal(A.n_rows, 1))
    ref, out = both(S, h, vals, b, S.cg_opts(rtol=1e-9, method="bicgstab"))
    check_equal(ref, out)
    monkeypatch.setenv("SLA_BAND_MIN_STRIDE", "300")
    P = W.poisson5(300)
    hp = S.csr_create(dev(P.row_ptr), dev(P.col), symmetric=True)
    assert S.csr_analysis(hp)["band_stride"] == 300
    ref, out = both(S, hp, dev(P.vals), dev(W.rhs_normal(P.n_rows, 2)), S.cg_opts(rtol=1e-10))
    check_equal(ref, out)


def test_noalloc_refuses_a_problem_beyond_the_scratch(S):
    from differentiable_sparse_linear_spmv_amd import _lib as L
    n = 2_000_000   # 4 vectors of 16 MB: past the 50 MiB scratch
    rp = torch.arange(n + 1, dtype=torch.int32, device="cuda")
    col = torch.arange(n, dtype=torch.int32, device="cuda")
    h = S.csr_create(rp, col, symmetric=True)
    vals = torch.full((n,), 2.0, dtype=torch.float64, device="cuda")
    b = torch.ones(n, dtype=torch.float64, device="cuda")
    x = torch.zeros_like(b)
    info = S.info_buffer(1, b.device)
    with pytest.raises(L.SlaError) as e:
        S.solve_noalloc(h, vals, b, S.cg_opts(rtol=1e-10), x, info)
    assert e.value.status == L.SLA_ERR_INVALID_ARG and "scratch" in str(e.value)
    assert torch.count_nonzero(x).item() == 0   # nothing ran
    # the same handle still solves through sla_solve (diagonal 2: one iteration)
    xs, inf = S.solve(h, vals, b, S.cg_opts(rtol=1e-10))
    assert S.read_info(inf)[0]["iterations"] == 1 and torch.allclose(xs, b / 2)
    del h
    gc.collect()
