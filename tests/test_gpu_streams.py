"""Determinism and stream placement of the eigensolvers, lists and batched solves,
through the C ABI: the same call twice gives the same bits (every reduction is summed
in a fixed order), and the same call enqueued on a side stream gives the same bits as
on the default stream (all work and every host wait go to the caller's stream)."""
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


def outputs(S):
    """Run every entry point once on the current stream; return host copies."""
    A, b, _ = W.varcoef_poisson5(90, seed=4)
    h = S.csr_create(dev(A.row_ptr), dev(A.col), symmetric=True)
    vals = dev(A.vals)
    x, info = S.solve(h, vals, dev(b), S.cg_opts(rtol=1e-10))
    gb, gv, _ = S.solve_backward(h, vals, x, x.clone(), S.cg_opts(rtol=1e-10))
    ev, U, _ = S.eigsh(h, vals, 4, dev(b), tol=1e-10)
    et, Ut, _ = S.eigsh(h, vals, 4, dev(b), tol=1e-10, max_dim=16, max_iter=5000)
    X0 = np.stack([W.rhs_normal(A.n_rows, 20 + r) for r in range(4)])
    el, Ul, _ = S.lobpcg(h, vals, 4, dev(X0), tol=1e-8, jacobi=True, which="smallest")
    F, bf = W.fem_p1_batched(nv=70, B=16, seed=1)          # grouped batch (span >= 4096)
    hf = S.csr_create(dev(F.row_ptr), dev(F.col), symmetric=True)
    xf, _ = S.solve(hf, dev(F.vals), dev(bf), S.cg_opts(rtol=1e-9))
    items = [W.poisson5(30), W.poisson5(45)]
    hl = S.list_create([dev(P.row_ptr) for P in items], [dev(P.col) for P in items], symmetric=True)
    xl, _ = S.list_solve(hl, [dev(P.vals) for P in items], [dev(W.rhs_normal(P.n_rows, 7)) for P in items],
                         S.cg_opts(rtol=1e-10))
    torch.cuda.current_stream().synchronize()
    return [t.cpu().numpy() for t in [x, gb, gv, ev, U, et, Ut, el, Ul, xf] + list(xl)]


def test_repeatable_to_the_bit(S):
    a = outputs(S)
    b = outputs(S)
    for i, (u, v) in enumerate(zip(a, b)):
        assert np.array_equal(u, v), i


def test_side_stream_gives_the_same_bits(S):
    ref = outputs(S)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        got = outputs(S)
    side.synchronize()
    for i, (u, v) in enumerate(zip(ref, got)):
        assert np.array_equal(u, v), i


def test_polling_interval_changes_nothing(S):
    # the host checks the stop word (CG) or the Ritz pairs (Lanczos) once per chunk of
    # iterations; work enqueued past the stop is discarded, so the chunk size must not
    # change a bit of the results or the counts
    A, b, _ = W.varcoef_poisson5(70, seed=9)
    h = S.csr_create(dev(A.row_ptr), dev(A.col), symmetric=True)
    vals = dev(A.vals)
    ref = None
    for every in (1, 5, 32, 200):
        o = S.cg_opts(rtol=1e-10, check_every=every)
        x, info = S.solve(h, vals, dev(b), o)
        ev, U, einfo = S.eigsh(h, vals, 3, dev(b), tol=1e-10, check_every=every)
        out = (x.cpu().numpy(), ev.cpu().numpy(), U.cpu().numpy(), S.read_info(info)[0]["iterations"],
               einfo["iterations"])
        if ref is None:
            ref = out
            continue
        for u, v in zip(ref[:3], out[:3]):
            assert np.array_equal(u, v), every
        assert ref[3:] == out[3:], (every, ref[3:], out[3:])
