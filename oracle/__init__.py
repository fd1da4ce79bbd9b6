"""CPU oracle for the sparse CG solve and its adjoint -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library under
``differentiable_sparse_linear_spmv_amd``) never imports it, and the two share
no code: the arithmetic lives in ``sla_oracle.c`` (plain sequential C, fp64,
no fused multiply-add); this module only marshals numpy arrays through ctypes.

What it computes, from torch-sla (Differentiable Sparse Linear Algebra with
Adjoint Solvers and Sparse Tensor Parallelism for PyTorch):
  * ``spmv``              y = A x (paperpeel page, section 3.3: SpMV).
  * ``cg``                unpreconditioned Hestenes-Stiefel CG, x0 = 0
                          (paperpeel section 1; section 3.3 "Distributed Krylov
                          solvers" for the two inner products per iteration), or
                          with ``jacobi=True`` Jacobi-preconditioned CG (section
                          4.1, Table 3).
  * ``bicgstab``          van der Vorst's BiCGStab, x0 = 0, shadow residual b
                          (paperpeel sections 1 and 3.1: the nonsymmetric solver of
                          the iterative backends).
  * ``solve_backward``    A^T lambda = dL/dx, dL/db = lambda,
                          dL/dA_ij = -lambda_i x_j on the pattern (gist.science
                          Hindi / Japanese summaries, Methodology item 2,
                          linear-systems bullet).
  * ``matvec_backward``   for y = A x: dL/dx = A^T gy, dL/dA_ij = gy_i x_j.
  * ``transpose``         stable counting-sort transpose of the pattern.
  * ``eigsh`` (module oracle/eigsh.py)  Lanczos eigenpairs and the Hellmann-Feynman
                          gradient (paperpeel section 4.3, note to Table 5).
Every function is pinned (tests/test_oracle_pins.py, test_oracle_bicgstab.py,
test_oracle_eigsh.py); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

CONVERGED, MAX_ITER, NOT_SPD, NAN, BREAKDOWN = 0, 1, 2, 3, 4
METHODS = {"cg": 0, "jacobi": 1, "bicgstab": 2}
_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("SLA_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and (not os.path.exists(path)
                                   or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
            _build.build(force=True)
        L = C.CDLL(path)
        P = C.c_void_p
        i64, f64, i32 = C.c_int64, C.c_double, C.c_int
        L.orc_spmv.argtypes = [i64, P, P, P, P, P]
        L.orc_spmv.restype = None
        L.orc_spmv_transposed.argtypes = [i64, i64, P, P, P, P, P]
        L.orc_spmv_transposed.restype = None
        L.orc_dot.argtypes = [i64, P, P]
        L.orc_dot.restype = f64
        L.orc_cg.argtypes = [i64, P, P, P, P, P, f64, f64, i64, i32, P, P, P, P, P]
        L.orc_cg.restype = i32
        L.orc_pcg_jacobi.argtypes = [i64, P, P, P, P, P, f64, f64, i64, i32, P, P, P, P, P]
        L.orc_pcg_jacobi.restype = i32
        L.orc_bicgstab.argtypes = [i64, P, P, P, P, P, f64, f64, i64, i32, P, P, P, P, P]
        L.orc_bicgstab.restype = i32
        L.orc_transpose.argtypes = [i64, i64, P, P, P, P, P]
        L.orc_transpose.restype = None
        L.orc_pattern_outer.argtypes = [i64, P, P, f64, P, P, P]
        L.orc_pattern_outer.restype = None
        L.orc_solve_backward.argtypes = [i64, P, P, P, i32, P, P, f64, f64, i64, i32, i32, P, P, P,
                                         P, P, P]
        L.orc_solve_backward.restype = i32
        L.orc_cg_timing.argtypes = [i64, P, P, P, P, P, i64, i32, P, P, P, i32]
        L.orc_cg_timing.restype = i32
        L.orc_bicgstab_timing.argtypes = [i64, P, P, P, P, P, i64, i32, P, P, P, P, P, P, i32]
        L.orc_bicgstab_timing.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _pattern(A):
    rp = np.ascontiguousarray(A.row_ptr, dtype=np.int64)
    col = np.ascontiguousarray(A.col, dtype=np.int32)
    return rp, col


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def spmv(A, x, vals=None) -> np.ndarray:
    rp, col = _pattern(A)
    v = _f64(A.vals if vals is None else vals)
    x = _f64(x)
    y = np.empty(A.n_rows, np.float64)
    lib().orc_spmv(A.n_rows, _p(rp), _p(col), _p(v), _p(x), _p(y))
    return y


def spmv_transposed(A, x, vals=None) -> np.ndarray:
    rp, col = _pattern(A)
    v = _f64(A.vals if vals is None else vals)
    x = _f64(x)
    y = np.empty(A.n_cols, np.float64)
    lib().orc_spmv_transposed(A.n_rows, A.n_cols, _p(rp), _p(col), _p(v), _p(x), _p(y))
    return y


def dot(a, b) -> float:
    a, b = _f64(a), _f64(b)
    return float(lib().orc_dot(a.shape[0], _p(a), _p(b)))


def cg(A, b, rtol=1e-10, atol=0.0, max_iter=100000, fixed=False, vals=None, history=False,
       jacobi=False, method=None):
    """Returns dict(x, iterations, state, res_norm, rhs_norm[, history]).  jacobi: the
    Jacobi-preconditioned variant (orc_pcg_jacobi); method="bicgstab": orc_bicgstab."""
    method = method or ("jacobi" if jacobi else "cg")
    rp, col = _pattern(A)
    v = _f64(A.vals if vals is None else vals)
    b = _f64(b)
    n = A.n_rows
    x = np.empty(n, np.float64)
    work = np.empty(5 * max(n, 1), np.float64)
    it, res, rhs = C.c_int64(0), C.c_double(0), C.c_double(0)
    hist = np.full(max_iter + 1, np.nan) if history else None
    fn = {"cg": lib().orc_cg, "jacobi": lib().orc_pcg_jacobi, "bicgstab": lib().orc_bicgstab}[method]
    st = fn(n, _p(rp), _p(col), _p(v), _p(b), _p(x), rtol, atol, max_iter,
                      1 if fixed else 0, _p(work), C.byref(it), C.byref(res), C.byref(rhs),
                      _p(hist) if history else None)
    out = dict(x=x, iterations=int(it.value), state=int(st), res_norm=float(res.value),
               rhs_norm=float(rhs.value))
    if history:
        out["history"] = hist[: it.value + 1].copy()
    return out


def bicgstab(A, b, **kw):
    """BiCGStab (orc_bicgstab); same arguments and result as :func:`cg`."""
    return cg(A, b, method="bicgstab", **kw)


def transpose(A):
    """Returns (row_ptr_t int64 [n_cols+1], col_t int32 [nnz], perm int64 [nnz])."""
    rp, col = _pattern(A)
    nnz = A.nnz
    rpt = np.empty(A.n_cols + 1, np.int64)
    ct = np.empty(max(nnz, 1), np.int32)
    perm = np.empty(max(nnz, 1), np.int64)
    lib().orc_transpose(A.n_rows, A.n_cols, _p(rp), _p(col), _p(rpt), _p(ct), _p(perm))
    return rpt, ct[:nnz], perm[:nnz]


def pattern_outer(A, u, v, sign=1.0) -> np.ndarray:
    rp, col = _pattern(A)
    u, v = _f64(u), _f64(v)
    g = np.empty(A.nnz, np.float64)
    lib().orc_pattern_outer(A.n_rows, _p(rp), _p(col), float(sign), _p(u), _p(v), _p(g))
    return g


def solve_backward(A, x, g, symmetric=True, rtol=1e-10, atol=0.0, max_iter=100000,
                   fixed=False, vals=None, jacobi=False, method=None):
    """Returns dict(lam (= dL/db), gvals (= dL/dvals), iterations, state, res_norm, rhs_norm).
    The adjoint solve uses the forward's method: "cg", "jacobi" or "bicgstab"."""
    method = method or ("jacobi" if jacobi else "cg")
    rp, col = _pattern(A)
    v = _f64(A.vals if vals is None else vals)
    x, g = _f64(x), _f64(g)
    n = A.n_rows
    lam = np.empty(n, np.float64)
    gv = np.empty(A.nnz, np.float64)
    work = np.empty(5 * max(n, 1), np.float64)
    it, res, rhs = C.c_int64(0), C.c_double(0), C.c_double(0)
    st = lib().orc_solve_backward(n, _p(rp), _p(col), _p(v), 1 if symmetric else 0, _p(x),
                                  _p(g), rtol, atol, max_iter, 1 if fixed else 0,
                                  METHODS[method], _p(lam),
                                  _p(gv), _p(work), C.byref(it), C.byref(res), C.byref(rhs))
    return dict(lam=lam, gvals=gv, iterations=int(it.value), state=int(st),
                res_norm=float(res.value), rhs_norm=float(rhs.value))


def matvec_backward(A, x, gy, vals=None):
    """Backward of y = A x: returns (gx = A^T gy, gvals_k = gy[row(k)] * x[col(k)])."""
    gx = spmv_transposed(A, gy, vals=vals)
    gv = pattern_outer(A, gy, x, sign=1.0)
    return gx, gv


def solve_batched(A, b, **kw):
    """Independent CG per system of a shared-pattern batch (vals [B, nnz], b [B, n])."""
    return [cg(A, b[s], vals=A.vals[s], **kw) for s in range(A.vals.shape[0])]


def solve_backward_batched(A, x, g, **kw):
    return [solve_backward(A, x[s], g[s], vals=A.vals[s], **kw) for s in range(A.vals.shape[0])]


def cg_timing(A, b, iters, threads, adjoint=True, vals=None):
    """The CPU baseline's timing mode (orc_cg_timing): `iters` fixed CG iterations on
    `threads` OpenMP threads, then (adjoint) the backward pass of L = 0.5 |x|^2 on a
    symmetric A with the same budget.  Returns dict(x, lam, gvals, threads)."""
    rp, col = _pattern(A)
    v = _f64(A.vals if vals is None else vals)
    b = _f64(b)
    n = A.n_rows
    x = np.empty(n, np.float64)
    lam = np.empty(n, np.float64)
    gv = np.empty(max(A.nnz, 1), np.float64)
    work = np.empty(4 * max(n, 1), np.float64)
    nt = lib().orc_cg_timing(n, _p(rp), _p(col), _p(v), _p(b), _p(x), int(iters), 1 if adjoint else 0,
                             _p(lam), _p(gv), _p(work), int(threads))
    return dict(x=x, lam=lam, gvals=gv[:A.nnz], threads=int(nt))


def bicgstab_timing(A, b, iters, threads, adjoint=True, vals=None):
    """The CPU baseline's BiCGStab timing mode (orc_bicgstab_timing): `iters` fixed
    iterations of orc_bicgstab's steps on `threads` OpenMP threads, then (adjoint) the
    same on A^T with right-hand side x and the gradient on A's pattern.  Returns
    dict(x, lam, gvals, threads)."""
    rp, col = _pattern(A)
    v = _f64(A.vals if vals is None else vals)
    b = _f64(b)
    n = A.n_rows
    rpt, ct, perm = transpose(A)
    vt = np.ascontiguousarray(v[perm]) if A.nnz > 0 else np.zeros(1)
    x = np.empty(n, np.float64)
    lam = np.empty(n, np.float64)
    gv = np.empty(max(A.nnz, 1), np.float64)
    work = np.empty(6 * max(n, 1), np.float64)
    nt = lib().orc_bicgstab_timing(n, _p(rp), _p(col), _p(v), _p(b), _p(x), int(iters), 1 if adjoint else 0,
                                   _p(rpt), _p(ct), _p(vt), _p(lam), _p(gv), _p(work), int(threads))
    return dict(x=x, lam=lam, gvals=gv[:A.nnz], threads=int(nt))
