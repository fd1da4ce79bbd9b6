"""The adjoint's memory claim, on the GPU: a solve and its backward through
SparseTensor hold O(n + nnz) device memory whatever the number of CG iterations k,
and the loss's autograd graph holds exactly one solve node (paperpeel page, section
3.2.3 "Complexity" and Table 2; section 4.2 "Adjoint vs. Naive Backpropagation",
Results: the adjoint's backward memory stays flat from k = 10 to k = 5000 on a
5-point Poisson system with nnz = 3.2e6).

The library's device memory goes through torch's caching allocator here
(use_torch_allocator), so torch.cuda.max_memory_allocated() sees the workspaces too.
"""
import gc

import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N = 800   # 640,000 unknowns, nnz = 3,196,800: the size of the pages' memory experiment


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differentiable_sparse_linear_spmv_amd as S
    S.use_torch_allocator(True)
    yield S
    S.use_torch_allocator(False)


def graph_nodes(t):
    """Names of every node reachable from t.grad_fn (each node once).  The visited
    nodes are kept alive, so that no id() is reused by a later wrapper object."""
    seen, keep, stack, names = set(), [], [t.grad_fn], []
    while stack:
        f = stack.pop()
        if f is None or id(f) in seen:
            continue
        seen.add(id(f))
        keep.append(f)
        names.append(type(f).__name__)
        stack.extend(g for g, _ in f.next_functions)
    return names


def one_run(S, rp, col, vals0, b0, k):
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    vals = vals0.clone().requires_grad_(True)
    b = b0.clone().requires_grad_(True)
    A = S.SparseTensor(rp, col, vals, symmetric=True)
    x = A.solve(b, rtol=0.0, max_iter=k, fixed=True)
    loss = 0.5 * (x * x).sum()
    names = graph_nodes(loss)
    loss.backward()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    ws = S.csr_info(A.handle)["workspace_bytes"]
    it = S.read_info(A.last_info)[0]["iterations"]
    bit = S.read_info(A.last_backward_info)[0]["iterations"]
    g = (vals.grad.norm().item(), b.grad.norm().item())
    del A, x, loss, vals, b
    gc.collect()
    torch.cuda.synchronize()
    return dict(peak=peak, ws=ws, names=names, it=it, bit=bit, g=g)


def test_backward_memory_flat_in_k_and_one_graph_node(S):
    Ah = W.poisson5(N)
    rp, col = torch.from_numpy(Ah.row_ptr).cuda(), torch.from_numpy(Ah.col).cuda()
    vals0 = torch.from_numpy(Ah.vals).cuda()
    b0 = torch.from_numpy(W.rhs_normal(Ah.n_rows, 0)).cuda()
    n, nnz = Ah.n_rows, Ah.nnz
    short = one_run(S, rp, col, vals0, b0, 10)
    long_ = one_run(S, rp, col, vals0, b0, 5000)
    print(f"\nn={n} nnz={nnz}: peak {short['peak'] / 2**20:.1f} MiB at k=10, {long_['peak'] / 2**20:.1f} MiB "
          f"at k=5000; workspace {short['ws'] / 2**20:.1f} MiB; graph {long_['names']}", flush=True)
    assert (short["it"], short["bit"]) == (10, 10)
    assert (long_["it"], long_["bit"]) == (5000, 5000)
    # flat in k: the same peak and the same workspace, to the byte
    assert long_["peak"] == short["peak"], (short["peak"], long_["peak"])
    assert long_["ws"] == short["ws"]
    # O(n + nnz): the values' gradient and copy (2 x 8 nnz), the pattern's offsets
    # (2 nnz), and a bounded number of n-vectors (b, x, r, p, p', q, lambda, dL/dx,
    # the gradients' temporaries) -- nothing per iteration
    assert long_["peak"] <= 18 * nnz + 8 * n * 16, long_["peak"]
    # one solve node whatever k, and a graph of a few nodes in all
    for r in (short, long_):
        assert r["names"].count("_SolveFnBackward") == 1, r["names"]
        assert len(r["names"]) <= 6, r["names"]
    assert sorted(short["names"]) == sorted(long_["names"])
    assert all(np.isfinite(v) and v > 0 for v in long_["g"])
