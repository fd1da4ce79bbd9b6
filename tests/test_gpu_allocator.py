"""The library's device memory through a caller's allocator (sla_set_allocator),
through the C ABI: torch's caching allocator holds the workspaces while a handle
lives, the results are those of the hipMalloc path bit for bit (the same kernels on
the same data), and every block goes back through the allocator that made it, also
after the allocator has been switched back.
"""
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
    yield S
    S.use_torch_allocator(False)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def run(S, A, b, X0):
    h = S.csr_create(dev(A.row_ptr), dev(A.col), symmetric=True)
    vals = dev(A.vals)
    x, _ = S.solve(h, vals, dev(b), S.cg_opts(rtol=1e-10))
    gb, gv, _ = S.solve_backward(h, vals, x, x.clone(), S.cg_opts(rtol=1e-10))
    ev, U, _ = S.eigsh(h, vals, 3, dev(b), tol=1e-10)
    ew, V, _ = S.lobpcg(h, vals, 3, dev(X0), tol=1e-8)
    torch.cuda.synchronize()
    return h, [t.cpu().numpy() for t in (x, gb, gv, ev, U, ew, V)]


def test_handle_outlives_the_switch(S):
    # blocks from torch's allocator, the allocator switched back, then the handle
    # destroyed: its blocks still go back to torch (the callbacks stay alive)
    base = torch.cuda.memory_allocated()
    S.use_torch_allocator(True)
    A = W.poisson5(40)
    h = S.csr_create(dev(A.row_ptr), dev(A.col), symmetric=True)
    x, info = S.solve(h, dev(A.vals), dev(W.rhs_normal(A.n_rows, 3)), S.cg_opts(rtol=1e-8))
    S.use_torch_allocator(False)
    gc.collect()
    del h, x, info
    gc.collect()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() <= base


def test_torch_allocator_holds_the_workspaces(S):
    A, b, _ = W.varcoef_poisson5(60, seed=2)
    X0 = np.stack([W.rhs_normal(A.n_rows, 5 + r) for r in range(3)])
    S.use_torch_allocator(False)
    h, ref = run(S, A, b, X0)
    del h
    gc.collect()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    S.use_torch_allocator(True)
    h, out = run(S, A, b, X0)
    held = torch.cuda.memory_allocated() - base
    # at least the CG workspace (4 vectors) and the LOBPCG block pool (43 vectors)
    assert held >= 8 * A.n_rows * (4 + 43), held
    for r, o in zip(ref, out):
        assert np.array_equal(r, o)
    del h
    gc.collect()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() - base <= 8 * A.n_rows * 4   # only the results remain
    S.use_torch_allocator(False)


def test_blocks_return_to_their_allocator(S):
    from differentiable_sparse_linear_spmv_amd import _lib as L
    calls = {"alloc": 0, "free": 0}

    def _alloc(size, stream, ctx):
        calls["alloc"] += 1
        return torch.cuda.caching_allocator_alloc(int(size))

    def _free(ptr, stream, ctx):
        calls["free"] += 1
        torch.cuda.caching_allocator_delete(ptr)

    cbs = (L.ALLOC_FN(_alloc), L.FREE_FN(_free))
    lib = L.load()
    assert lib.sla_set_allocator(cbs[0], cbs[1], None) == 0
    A = W.poisson5(50)
    b = W.rhs_normal(A.n_rows, 1)
    h = S.csr_create(dev(A.row_ptr), dev(A.col), symmetric=False)   # the adjoint builds a transpose
    x, _ = S.solve(h, dev(A.vals), dev(b), S.cg_opts(rtol=1e-8))
    S.solve_backward(h, dev(A.vals), x, x.clone(), S.cg_opts(rtol=1e-8))
    torch.cuda.synchronize()
    # blocks live in the handle (workspace, transpose, transposed values); create-time
    # validation and transpose scratch have come and gone already
    live = calls["alloc"] - calls["free"]
    assert live >= 3, calls
    # switch back to hipMalloc while the handle holds blocks of the callbacks: its
    # destruction must still free them through the callbacks
    assert lib.sla_set_allocator(L.ALLOC_FN(), L.FREE_FN(), None) == 0
    del h
    gc.collect()
    torch.cuda.synchronize()
    assert calls["free"] == calls["alloc"], calls


def test_failing_allocator_reports_oom_and_leaks_nothing(S):
    # An allocator that returns NULL at its N-th call, for every N that a create +
    # solve + adjoint on a non-symmetric handle reaches (validation scratch, workspace,
    # the transpose, its scratch and offsets, the transposed values).  Each failing call
    # reports SLA_ERR_OOM; the handle it leaves (if create succeeded) then finishes the
    # same run bit for bit once allocation works again, so a half-built transpose left
    # nothing behind; and after the handle is gone every block has come back.
    from differentiable_sparse_linear_spmv_amd import _lib as L
    lib = L.load()
    A = W.poisson5(30)     # declared non-symmetric: the adjoint runs on the device transpose
    b = W.rhs_normal(A.n_rows, 2)
    state = {"calls": 0, "fail_at": 0, "live": {}, "bad_free": 0}

    def _alloc(size, stream, ctx):
        state["calls"] += 1
        if state["calls"] == state["fail_at"]:
            return None
        p = torch.cuda.caching_allocator_alloc(int(size))
        state["live"][p] = int(size)
        return p

    def _free(ptr, stream, ctx):
        if state["live"].pop(ptr, None) is None:
            state["bad_free"] += 1
            return
        torch.cuda.caching_allocator_delete(ptr)

    cbs = (L.ALLOC_FN(_alloc), L.FREE_FN(_free))
    assert lib.sla_set_allocator(cbs[0], cbs[1], None) == 0
    opts = S.cg_opts(rtol=1e-10)
    rp, col, vals, bd = dev(A.row_ptr), dev(A.col), dev(A.vals), dev(b)

    def full_run(h):
        x, _ = S.solve(h, vals, bd, opts)
        gb, gv, _ = S.solve_backward(h, vals, x, x.clone(), opts)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in (x, gb, gv)]

    try:
        h = S.csr_create(rp, col, symmetric=False)
        ref = full_run(h)
        total = state["calls"]
        del h
        gc.collect()
        torch.cuda.synchronize()
        assert not state["live"] and total >= 5, (state, total)
        failed = 0
        for n_fail in range(1, total + 1):
            state.update(calls=0, fail_at=n_fail)
            h = None
            try:
                h = S.csr_create(rp, col, symmetric=False)
                full_run(h)
            except L.SlaError as e:
                assert e.status == L.SLA_ERR_OOM, (n_fail, str(e))
                failed += 1
            state["fail_at"] = 0
            if h is not None:   # the handle survives a failed call and completes the run
                out = full_run(h)
                for r, o in zip(ref, out):
                    assert np.array_equal(r, o), n_fail
            del h
            gc.collect()
            torch.cuda.synchronize()
            assert not state["live"], (n_fail, state["live"])
        assert failed == total, (failed, total)
        assert state["bad_free"] == 0
    finally:
        assert lib.sla_set_allocator(L.ALLOC_FN(), L.FREE_FN(), None) == 0
