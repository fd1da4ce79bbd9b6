"""Python surface of the HIP library: C-ABI calls with the same names, and the
SparseTensor / autograd wrappers of torch-sla's API (.matvec, .solve with
gradients to the values and to b).

torch-sla (Differentiable Sparse Linear Algebra with Adjoint Solvers and Sparse
Tensor Parallelism for PyTorch), paperpeel page, section 3.1: every operation is
one torch.autograd.Function whose forward calls the solver under no_grad and
stashes (A, x), and whose backward runs the adjoint solve -- one graph node and
O(n + nnz) memory whatever the iteration count (section 3.2).  A SparseTensor is
one matrix or a batch of matrices that share one pattern ("Typed sparse-tensor
hierarchy").  Here the forward and backward are the C-ABI calls sla_solve and
sla_solve_backward; this module only marshals tensors (device pointers, sizes,
torch's current HIP stream) and never computes on the host.
"""
from __future__ import annotations

import ctypes as C
import warnings

import torch

from . import _lib as L
from ._lib import SlaCgInfo, SlaCgOpts, SlaEigInfo, SlaEigOpts, check

__all__ = [
    "csr_create", "csr_destroy", "csr_info", "csr_analysis", "matvec", "matvec_backward", "solve",
    "solve_noalloc", "info_buffer",
    "solve_backward", "cg_opts", "read_info", "eigsh", "eigsh_backward", "list_create", "list_solve",
    "list_solve_backward", "SparseTensor", "SparseTensorList", "timing",
]


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, numel: int, device) -> None:
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


class Handle:
    """Owns an sla_csr* and keeps the borrowed row_ptr / col tensors alive."""

    def __init__(self, ptr: int, row_ptr: torch.Tensor, col: torch.Tensor, n_rows: int,
                 n_cols: int, symmetric: bool):
        self.ptr = C.c_void_p(ptr)
        self.row_ptr, self.col = row_ptr, col
        self.n_rows, self.n_cols, self.nnz = n_rows, n_cols, int(col.numel())
        self.symmetric = symmetric
        self.device = row_ptr.device

    def __del__(self):
        p = getattr(self, "ptr", None)
        if p is not None and p.value:
            try:
                L.load().sla_csr_destroy(p)
            except Exception:
                pass
            self.ptr = C.c_void_p(0)


def csr_create(row_ptr: torch.Tensor, col: torch.Tensor, n_cols: int | None = None,
               symmetric: bool = False, eager_transpose: bool = False) -> Handle:
    """sla_csr_create: validate the pattern on the device and analyse it."""
    lib = L.load()
    if row_ptr.dtype not in (torch.int32, torch.int64):
        raise ValueError("row_ptr must be int32 or int64")
    if col.dtype != torch.int32:
        raise ValueError("col must be int32")
    if not row_ptr.is_cuda or col.device != row_ptr.device:
        raise ValueError("row_ptr and col must be on the same GPU")
    row_ptr, col = row_ptr.contiguous(), col.contiguous()
    n_rows = row_ptr.numel() - 1
    n_cols = n_rows if n_cols is None else int(n_cols)
    flags = (L.SLA_SYMMETRIC if symmetric else 0) | (L.SLA_EAGER_TRANSPOSE if eager_transpose else 0)
    out = C.c_void_p()
    with torch.cuda.device(row_ptr.device):
        check(lib.sla_csr_create(C.byref(out), n_rows, n_cols, col.numel(), row_ptr.data_ptr(),
                                 32 if row_ptr.dtype == torch.int32 else 64,
                                 col.data_ptr() if col.numel() else None, flags,
                                 _stream(row_ptr.device)))
    return Handle(out.value, row_ptr, col, n_rows, n_cols, symmetric)


def csr_destroy(h: Handle) -> None:
    h.__del__()


def csr_info(h: Handle) -> dict:
    lib = L.load()
    a, b, c, w = C.c_int64(), C.c_int64(), C.c_int64(), C.c_int64()
    bits, fl = C.c_int32(), C.c_uint32()
    check(lib.sla_csr_info(h.ptr, C.byref(a), C.byref(b), C.byref(c), C.byref(bits),
                           C.byref(fl), C.byref(w)))
    return dict(n_rows=a.value, n_cols=b.value, nnz=c.value, row_ptr_bits=bits.value,
                flags=fl.value, workspace_bytes=w.value)


def csr_analysis(h: Handle) -> dict:
    lib = L.load()
    rm, tm, cap, band, split = C.c_int32(), C.c_int32(), C.c_int32(), C.c_int64(), C.c_int32()
    check(lib.sla_csr_analysis(h.ptr, C.byref(rm), C.byref(tm), C.byref(cap), C.byref(band),
                               C.byref(split)))
    cb, nd, gw = C.c_int32(), C.c_int32(), C.c_int32()
    check(lib.sla_csr_col_bits(h.ptr, C.byref(cb)))
    check(lib.sla_csr_diagonals(h.ptr, C.byref(nd)))
    check(lib.sla_csr_group_window(h.ptr, C.byref(gw)))
    return dict(row_max=rm.value, tile_max=tm.value, spmv_cap=cap.value, band_stride=band.value,
                split=bool(split.value), col_bits=cb.value, diagonals=nd.value, group_window=gw.value)


def _batch_of(vals: torch.Tensor, nnz: int) -> int:
    if vals.dim() == 1:
        return 1
    if vals.dim() == 2 and vals.shape[1] == nnz:
        return int(vals.shape[0])
    raise ValueError(f"vals must be [nnz] or [batch, nnz] (got {tuple(vals.shape)})")


def matvec(h: Handle, vals: torch.Tensor, x: torch.Tensor, y: torch.Tensor | None = None):
    """sla_matvec: y = A x for every system of the batch."""
    B = _batch_of(vals, h.nnz)
    _need(vals, "vals", torch.float64, B * h.nnz, h.device)
    _need(x, "x", torch.float64, B * h.n_cols, h.device)
    if y is None:
        y = torch.empty((B, h.n_rows) if vals.dim() == 2 else (h.n_rows,), dtype=torch.float64,
                        device=h.device)
    _need(y, "y", torch.float64, B * h.n_rows, h.device)
    check(L.load().sla_matvec(h.ptr, B, _ptr(vals), _ptr(x), _ptr(y), _stream(h.device)))
    return y


def matvec_backward(h: Handle, vals: torch.Tensor, x: torch.Tensor, gy: torch.Tensor,
                    need_gx: bool = True, need_gvals: bool = True):
    """sla_matvec_backward: (gx = A^T gy, gvals = gy[row] * x[col])."""
    B = _batch_of(vals, h.nnz)
    _need(gy, "gy", torch.float64, B * h.n_rows, h.device)
    gx = gv = None
    if need_gx:
        _need(vals, "vals", torch.float64, B * h.nnz, h.device)
        gx = torch.empty((B, h.n_cols) if vals.dim() == 2 else (h.n_cols,), dtype=torch.float64,
                         device=h.device)
    if need_gvals:
        _need(x, "x", torch.float64, B * h.n_cols, h.device)
        gv = torch.empty_like(vals)
    check(L.load().sla_matvec_backward(h.ptr, B, _ptr(vals), _ptr(x), _ptr(gy), _ptr(gx),
                                       _ptr(gv), _stream(h.device)))
    return gx, gv


def cg_opts(rtol=1e-10, atol=0.0, max_iter=100000, fixed=False, check_every=0,
            residual_history: torch.Tensor | None = None, jacobi: bool = False,
            method: str = "cg") -> SlaCgOpts:
    """Solver options.  method: "cg" (with jacobi=True, Jacobi-preconditioned) or
    "bicgstab" (nonsymmetric systems; the adjoint then runs BiCGStab on A^T)."""
    if method not in ("cg", "bicgstab"):
        raise ValueError(f"unknown method {method!r} (expected 'cg' or 'bicgstab')")
    flags = ((L.SLA_FIXED_ITERS if fixed else 0) | (L.SLA_JACOBI if jacobi else 0)
             | (L.SLA_BICGSTAB if method == "bicgstab" else 0))
    return SlaCgOpts(float(rtol), float(atol), int(max_iter), int(check_every), flags,
                     residual_history.data_ptr() if residual_history is not None else None)


def _info_buffer(B: int, device) -> torch.Tensor:
    return torch.empty(B * C.sizeof(SlaCgInfo), dtype=torch.uint8, device=device)


def read_info(info: torch.Tensor) -> list[dict]:
    """Copy a device sla_cg_info array to the host (synchronises the stream)."""
    raw = info.cpu().numpy().tobytes()
    n = len(raw) // C.sizeof(SlaCgInfo)
    out = []
    for i in range(n):
        s = SlaCgInfo.from_buffer_copy(raw[i * 32:(i + 1) * 32])
        out.append(dict(iterations=s.iterations, res_norm=s.res_norm, rhs_norm=s.rhs_norm,
                        state=s.state, state_name=L.STATE_NAMES.get(s.state, str(s.state))))
    return out


def solve_noalloc(h: Handle, vals: torch.Tensor, b: torch.Tensor, opts: SlaCgOpts,
                  x: torch.Tensor, info: torch.Tensor):
    """sla_solve_noalloc: sla_solve with its workspace in the library's static device
    scratch (nothing allocated by the call).  The caller passes x and info (from
    info_buffer); calls that overlap on one GPU race."""
    B = _batch_of(vals, h.nnz)
    _need(vals, "vals", torch.float64, B * h.nnz, h.device)
    _need(b, "b", torch.float64, B * h.n_rows, h.device)
    _need(x, "x", torch.float64, B * h.n_rows, h.device)
    _need(info, "info", torch.uint8, B * C.sizeof(SlaCgInfo), h.device)
    check(L.load().sla_solve_noalloc(h.ptr, B, _ptr(vals), _ptr(b), _ptr(x), C.byref(opts), _ptr(info),
                                     _stream(h.device)))
    return x, info


def info_buffer(batch: int, device) -> torch.Tensor:
    """A device buffer for `batch` sla_cg_info records."""
    return _info_buffer(batch, device)


def solve(h: Handle, vals: torch.Tensor, b: torch.Tensor, opts: SlaCgOpts,
          x: torch.Tensor | None = None, info: torch.Tensor | None = None):
    """sla_solve: CG from x0 = 0.  Returns (x, info) with info a device byte buffer."""
    B = _batch_of(vals, h.nnz)
    _need(vals, "vals", torch.float64, B * h.nnz, h.device)
    _need(b, "b", torch.float64, B * h.n_rows, h.device)
    if x is None:
        x = torch.empty_like(b)
    _need(x, "x", torch.float64, B * h.n_rows, h.device)
    if info is None:
        info = _info_buffer(B, h.device)
    check(L.load().sla_solve(h.ptr, B, _ptr(vals), _ptr(b), _ptr(x), C.byref(opts), _ptr(info),
                             _stream(h.device)))
    return x, info


def solve_backward(h: Handle, vals: torch.Tensor, x: torch.Tensor, gx: torch.Tensor,
                   opts: SlaCgOpts, need_gvals: bool = True, gb: torch.Tensor | None = None,
                   gvals: torch.Tensor | None = None, info: torch.Tensor | None = None):
    """sla_solve_backward: returns (gb = lambda, gvals = -lambda[row] x[col], info)."""
    B = _batch_of(vals, h.nnz)
    _need(vals, "vals", torch.float64, B * h.nnz, h.device)
    _need(gx, "gx", torch.float64, B * h.n_rows, h.device)
    if gb is None:
        gb = torch.empty_like(gx)
    _need(gb, "gb", torch.float64, B * h.n_rows, h.device)
    if need_gvals:
        _need(x, "x", torch.float64, B * h.n_rows, h.device)
        if gvals is None:
            gvals = torch.empty_like(vals)
        _need(gvals, "gvals", torch.float64, B * h.nnz, h.device)
    else:
        gvals = None
    if info is None:
        info = _info_buffer(B, h.device)
    check(L.load().sla_solve_backward(h.ptr, B, _ptr(vals), _ptr(x), _ptr(gx), _ptr(gb),
                                      _ptr(gvals), C.byref(opts), _ptr(info), _stream(h.device)))
    return gb, gvals, info


def eigsh(h: Handle, vals: torch.Tensor, k: int, v0: torch.Tensor, which: str = "largest",
          tol: float = 1e-10, max_dim: int = 0, check_every: int = 0, max_iter: int = 0, keep: int = 0):
    """sla_eigsh: k extreme eigenpairs by Lanczos (thick-restarted when max_iter > max_dim).
    Returns (evals [k], evecs [k, n], info)."""
    if which not in ("largest", "smallest"):
        raise ValueError(f"which must be 'largest' or 'smallest' (got {which!r})")
    _need(vals, "vals", torch.float64, h.nnz, h.device)
    _need(v0, "v0", torch.float64, h.n_rows, h.device)
    evals = torch.empty(k, dtype=torch.float64, device=h.device)
    evecs = torch.empty((k, h.n_rows), dtype=torch.float64, device=h.device)
    opts = SlaEigOpts(float(tol), int(max_dim), L.SLA_EIG_LARGEST if which == "largest" else L.SLA_EIG_SMALLEST,
                      int(check_every), int(max_iter), int(keep), 0)
    info = SlaEigInfo()
    check(L.load().sla_eigsh(h.ptr, _ptr(vals), int(k), _ptr(v0), _ptr(evals), _ptr(evecs), C.byref(opts),
                             C.byref(info), _stream(h.device)))
    return evals, evecs, dict(iterations=info.iterations, max_res=info.max_res, state=info.state,
                              restarts=info.restarts, state_name=L.STATE_NAMES.get(info.state, str(info.state)))


# Every callback pair ever registered stays alive: blocks they allocated are freed
# through them even after the allocator has been switched (a handle may outlive it).
_ALLOCATORS = []


def use_torch_allocator(enable: bool = True) -> None:
    """sla_set_allocator with torch's caching allocator (enable) or back to hipMalloc.
    The library's workspaces then count in torch.cuda.memory_allocated() and come from
    torch's pool on the current device and stream."""
    lib = L.load()
    if not enable:
        check(lib.sla_set_allocator(L.ALLOC_FN(), L.FREE_FN(), None))
        return

    def _alloc(size, stream, ctx):
        try:
            return torch.cuda.caching_allocator_alloc(int(size))
        except RuntimeError:   # out of memory: the library reports SLA_ERR_OOM
            return None

    def _free(ptr, stream, ctx):
        torch.cuda.caching_allocator_delete(ptr)

    cbs = (L.ALLOC_FN(_alloc), L.FREE_FN(_free))
    _ALLOCATORS.append(cbs)
    check(lib.sla_set_allocator(cbs[0], cbs[1], None))


def lobpcg(h: Handle, vals: torch.Tensor, k: int, X0: torch.Tensor, which: str = "largest", tol: float = 1e-8,
           max_iter: int = 0, jacobi: bool = False):
    """sla_lobpcg: k extreme eigenpairs by LOBPCG from the start block X0 [k, n]
    (jacobi: residuals preconditioned by diag(A)^-1).  Returns (evals [k], evecs [k, n], info)."""
    if which not in ("largest", "smallest"):
        raise ValueError(f"which must be 'largest' or 'smallest' (got {which!r})")
    _need(vals, "vals", torch.float64, h.nnz, h.device)
    _need(X0, "X0", torch.float64, k * h.n_rows, h.device)
    evals = torch.empty(k, dtype=torch.float64, device=h.device)
    evecs = torch.empty((k, h.n_rows), dtype=torch.float64, device=h.device)
    opts = SlaEigOpts(float(tol), 0, L.SLA_EIG_LARGEST if which == "largest" else L.SLA_EIG_SMALLEST, 0,
                      int(max_iter), 0, L.SLA_EIG_JACOBI if jacobi else 0)
    info = SlaEigInfo()
    check(L.load().sla_lobpcg(h.ptr, _ptr(vals), int(k), _ptr(X0), _ptr(evals), _ptr(evecs), C.byref(opts),
                              C.byref(info), _stream(h.device)))
    return evals, evecs, dict(iterations=info.iterations, max_res=info.max_res, state=info.state,
                              state_name=L.STATE_NAMES.get(info.state, str(info.state)))


def eigsh_backward(h: Handle, evecs: torch.Tensor, gevals: torch.Tensor, gvals: torch.Tensor | None = None):
    """sla_eigsh_backward: dL/dvals[e] = sum_r gevals[r] u_r[row(e)] u_r[col(e)]."""
    k = int(gevals.numel())
    _need(evecs, "evecs", torch.float64, k * h.n_rows, h.device)
    _need(gevals, "gevals", torch.float64, k, h.device)
    if gvals is None:
        gvals = torch.empty(h.nnz, dtype=torch.float64, device=h.device)
    _need(gvals, "gvals", torch.float64, h.nnz, h.device)
    check(L.load().sla_eigsh_backward(h.ptr, k, _ptr(evecs), _ptr(gevals), _ptr(gvals), _stream(h.device)))
    return gvals


class ListHandle:
    """Owns an sla_list* (items with distinct patterns, packed on the device)."""

    def __init__(self, ptr: int, n: list[int], nnz: list[int], symmetric: bool, device):
        self.ptr = C.c_void_p(ptr)
        self.n, self.nnz = n, nnz
        self.items = len(n)
        self.symmetric = symmetric
        self.device = device

    def __del__(self):
        try:
            if self.ptr:
                L.load().sla_list_destroy(self.ptr)
                self.ptr = C.c_void_p(0)
        except Exception:
            pass


def _ptr_array(ts) -> C.Array:
    return (C.c_void_p * len(ts))(*[None if t is None else t.data_ptr() for t in ts])


def list_create(row_ptrs: list[torch.Tensor], cols: list[torch.Tensor], symmetric: bool = False) -> ListHandle:
    """sla_list_create: items with their own square CSR patterns (same row-pointer dtype)."""
    if len(row_ptrs) != len(cols) or not row_ptrs:
        raise ValueError("need as many row_ptr as col tensors, at least one")
    dt = row_ptrs[0].dtype
    if dt not in (torch.int32, torch.int64) or any(r.dtype != dt for r in row_ptrs):
        raise ValueError("row pointers must all be int32 or all int64")
    dev = row_ptrs[0].device
    for r, c in zip(row_ptrs, cols):
        if r.device != dev or c.device != dev or c.dtype != torch.int32 or not (r.is_contiguous() and c.is_contiguous()):
            raise ValueError("row_ptr / col must be contiguous, on one device, col int32")
    n = [int(r.numel()) - 1 for r in row_ptrs]
    nnz = [int(c.numel()) for c in cols]
    ns = (C.c_int64 * len(n))(*n)
    zs = (C.c_int64 * len(nnz))(*nnz)
    out = C.c_void_p()
    flags = L.SLA_SYMMETRIC if symmetric else 0
    check(L.load().sla_list_create(C.byref(out), len(n), ns, zs, _ptr_array(row_ptrs),
                                   32 if dt == torch.int32 else 64, _ptr_array(cols), flags, _stream(dev)))
    h = ListHandle(out.value, n, nnz, symmetric, dev)
    h._keep = (row_ptrs, cols)
    return h


def list_col_bits(h: ListHandle) -> int:
    """sla_list_col_bits: 16 if the list's SpMV reads 16-bit column offsets, else 32."""
    cb = C.c_int32()
    check(L.load().sla_list_col_bits(h.ptr, C.byref(cb)))
    return cb.value


def list_solve(h: ListHandle, vals: list[torch.Tensor], b: list[torch.Tensor], opts: SlaCgOpts):
    """sla_list_solve: returns ([x_i], info) with info a device byte buffer [items]."""
    for i in range(h.items):
        _need(vals[i], f"vals[{i}]", torch.float64, h.nnz[i], h.device)
        _need(b[i], f"b[{i}]", torch.float64, h.n[i], h.device)
    x = [torch.empty_like(bi) for bi in b]
    info = _info_buffer(h.items, h.device)
    check(L.load().sla_list_solve(h.ptr, _ptr_array(vals), _ptr_array(b), _ptr_array(x), C.byref(opts),
                                  _ptr(info), _stream(h.device)))
    return x, info


def list_solve_backward(h: ListHandle, vals: list[torch.Tensor], x: list[torch.Tensor], gx: list[torch.Tensor],
                        opts: SlaCgOpts, need_gvals: bool = True):
    """sla_list_solve_backward: returns ([lambda_i], [gvals_i] or None, info)."""
    for i in range(h.items):
        _need(vals[i], f"vals[{i}]", torch.float64, h.nnz[i], h.device)
        _need(gx[i], f"gx[{i}]", torch.float64, h.n[i], h.device)
    gb = [torch.empty_like(g) for g in gx]
    gv = [torch.empty_like(v) for v in vals] if need_gvals else None
    info = _info_buffer(h.items, h.device)
    check(L.load().sla_list_solve_backward(h.ptr, _ptr_array(vals), _ptr_array(x) if need_gvals else None,
                                           _ptr_array(gx), _ptr_array(gb), _ptr_array(gv) if need_gvals else None,
                                           C.byref(opts), _ptr(info), _stream(h.device)))
    return gb, gv, info


class timing:
    """Per-kernel HIP-event timing inside the library (for measurement only)."""

    @staticmethod
    def enable(on: bool = True):
        check(L.load().sla_timing_enable(1 if on else 0))

    @staticmethod
    def reset():
        check(L.load().sla_timing_reset())

    @staticmethod
    def collect():
        check(L.load().sla_timing_collect())

    @staticmethod
    def query() -> dict:
        lib = L.load()
        out = {}
        for k, name in enumerate(L.KERNEL_NAMES):
            n, ms, by = C.c_int64(), C.c_double(), C.c_double()
            check(lib.sla_timing_query(k, C.byref(n), C.byref(ms)))
            check(lib.sla_timing_query_bytes(k, C.byref(by)))
            out[name] = dict(launches=n.value, total_ms=ms.value, bytes=by.value)
        return out


# ------------------------------------------------------------------------------ autograd
class _SolveFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, A, vals, b, opts_kw):
        opts = cg_opts(**opts_kw)
        x, info = solve(A.handle, vals.detach(), b.detach(), opts)
        A.last_info = info
        ctx.A, ctx.opts_kw = A, opts_kw
        ctx.save_for_backward(vals, x)
        return x

    @staticmethod
    def backward(ctx, gx):
        vals, x = ctx.saved_tensors
        A = ctx.A
        opts = cg_opts(**ctx.opts_kw)
        gb, gvals, info = solve_backward(A.handle, vals.detach(), x, gx.contiguous(), opts,
                                         need_gvals=ctx.needs_input_grad[1])
        A.last_backward_info = info
        return None, gvals, (gb if ctx.needs_input_grad[2] else None), None


class _EigshFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, A, vals, v0, kw):
        if kw["method"] == "lobpcg":
            evals, evecs, info = lobpcg(A.handle, vals.detach(), kw["k"], v0.detach(), which=kw["which"],
                                        tol=kw["tol"], max_iter=kw["max_iter"], jacobi=kw["jacobi"])
        else:
            evals, evecs, info = eigsh(A.handle, vals.detach(), kw["k"], v0.detach(), which=kw["which"],
                                       tol=kw["tol"], max_dim=kw["max_dim"], max_iter=kw["max_iter"],
                                       keep=kw["keep"])
        A.last_eig_info = info
        ctx.A = A
        ctx.save_for_backward(evecs)
        ctx.mark_non_differentiable(evecs)
        return evals, evecs

    @staticmethod
    def backward(ctx, gevals, _gevecs):
        (evecs,) = ctx.saved_tensors
        gvals = None
        if ctx.needs_input_grad[1]:
            gvals = eigsh_backward(ctx.A.handle, evecs, gevals.contiguous())
        return None, gvals, None, None


class _ListSolveFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, T, opts_kw, *tensors):
        k = T.handle.items
        vals, b = [t.detach() for t in tensors[:k]], [t.detach() for t in tensors[k:]]
        x, info = list_solve(T.handle, vals, b, cg_opts(**opts_kw))
        T.last_info = info
        ctx.T, ctx.opts_kw = T, opts_kw
        ctx.save_for_backward(*vals, *x)
        return tuple(x)

    @staticmethod
    def backward(ctx, *gx):
        T = ctx.T
        k = T.handle.items
        saved = ctx.saved_tensors
        vals, x = list(saved[:k]), list(saved[k:])
        need_v = any(ctx.needs_input_grad[2:2 + k])
        gx = [g.contiguous() if g is not None else torch.zeros_like(xi) for g, xi in zip(gx, x)]
        gb, gv, info = list_solve_backward(T.handle, vals, x, gx, cg_opts(**ctx.opts_kw), need_gvals=need_v)
        T.last_backward_info = info
        gvals = gv if need_v else [None] * k
        gbs = [g if ctx.needs_input_grad[2 + k + i] else None for i, g in enumerate(gb)]
        return (None, None, *gvals, *gbs)


class _MatvecFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, A, vals, x):
        y = matvec(A.handle, vals.detach(), x.detach())
        ctx.A = A
        ctx.save_for_backward(vals, x)
        return y

    @staticmethod
    def backward(ctx, gy):
        vals, x = ctx.saved_tensors
        gx, gv = matvec_backward(ctx.A.handle, vals.detach(), x.detach(), gy.contiguous(),
                                 need_gx=ctx.needs_input_grad[2],
                                 need_gvals=ctx.needs_input_grad[1])
        return None, gv, gx


class SparseTensor:
    """One CSR matrix, or a batch of matrices sharing one pattern (vals [B, nnz]).

    ``matvec(x)`` and ``solve(b)`` are differentiable with respect to ``vals`` and
    to ``x`` / ``b``; each is one autograd node.
    """

    def __init__(self, row_ptr: torch.Tensor, col: torch.Tensor, vals: torch.Tensor,
                 shape: tuple[int, int] | None = None, symmetric: bool = False):
        n_cols = None if shape is None else shape[1]
        self.handle = csr_create(row_ptr, col, n_cols=n_cols, symmetric=symmetric)
        self.vals = vals
        self.shape = (self.handle.n_rows, self.handle.n_cols)
        self.last_info = None
        self.last_backward_info = None
        self.last_eig_info = None

    @property
    def batch(self) -> int:
        return _batch_of(self.vals, self.handle.nnz)

    def matvec(self, x: torch.Tensor) -> torch.Tensor:
        return _MatvecFn.apply(self, self.vals, x)

    def solve(self, b: torch.Tensor, rtol=1e-10, atol=0.0, max_iter=100000, fixed=False,
              check: bool = False, jacobi: bool = False, method: str = "cg") -> torch.Tensor:
        kw = dict(rtol=rtol, atol=atol, max_iter=max_iter, fixed=fixed, jacobi=jacobi, method=method)
        x = _SolveFn.apply(self, self.vals, b, kw)
        if check:
            name = "BiCGStab" if method == "bicgstab" else "CG"
            for i, s in enumerate(read_info(self.last_info)):
                if s["state"] in (L.SLA_NOT_SPD, L.SLA_NAN, L.SLA_BREAKDOWN):
                    raise FloatingPointError(f"system {i}: {name} stopped with {s['state_name']}")
                if s["state"] == L.SLA_MAX_ITER and not fixed:
                    warnings.warn(f"system {i}: {name} reached max_iter={max_iter} "
                                  f"(|r|/|b| = {s['res_norm'] / max(s['rhs_norm'], 1e-300):.3e})")
        return x

    def eigsh(self, k: int = 6, which: str = "largest", tol: float = 1e-10, max_dim: int = 0,
              v0: torch.Tensor | None = None, max_iter: int = 0, keep: int = 0, method: str = "lanczos",
              jacobi: bool = False):
        """k extreme eigenpairs; the eigenvalues are differentiable with respect to vals
        (Hellmann-Feynman), the eigenvectors carry no gradient.
        method "lanczos": v0 is the start vector [n] (by default N(0, 1) from a
        generator seeded with 0 on the matrix's device); max_iter > max_dim: thick
        restart of a basis of max_dim vectors, keeping `keep` Ritz vectors, up to
        max_iter steps in all.
        method "lobpcg": v0 is the start block [k, n] (by default N(0, 1) as above);
        max_iter counts iterations (0: 1000); jacobi preconditions the residuals with
        diag(A)^-1 (for the smallest end).  Returns (evals [k], evecs [k, n])."""
        if method not in ("lanczos", "lobpcg"):
            raise ValueError(f"method must be 'lanczos' or 'lobpcg' (got {method!r})")
        if v0 is None:
            gen = torch.Generator(device=self.handle.device).manual_seed(0)
            shape = (k, self.handle.n_rows) if method == "lobpcg" else (self.handle.n_rows,)
            v0 = torch.randn(shape, dtype=torch.float64, device=self.handle.device, generator=gen)
        if jacobi and method != "lobpcg":
            raise ValueError("jacobi applies to method='lobpcg'")
        kw = dict(k=k, which=which, tol=tol, max_dim=max_dim, max_iter=max_iter, keep=keep, method=method,
                  jacobi=jacobi)
        return _EigshFn.apply(self, self.vals, v0, kw)

    def info(self, backward: bool = False) -> list[dict]:
        buf = self.last_backward_info if backward else self.last_info
        return [] if buf is None else read_info(buf)


class SparseTensorList:
    """A list of square sparse matrices with distinct patterns (the pages' SparseTensorList).

    ``solve([b_i])`` solves every item in one packed CG run on the device and is one
    autograd node, differentiable with respect to every ``vals_i`` and ``b_i``.
    """

    def __init__(self, row_ptrs: list[torch.Tensor], cols: list[torch.Tensor], vals: list[torch.Tensor],
                 symmetric: bool = False):
        self.handle = list_create(row_ptrs, cols, symmetric=symmetric)
        self.vals = list(vals)
        self.last_info = None
        self.last_backward_info = None

    def __len__(self) -> int:
        return self.handle.items

    def solve(self, b: list[torch.Tensor], rtol=1e-10, atol=0.0, max_iter=100000, fixed=False,
              jacobi: bool = False) -> list[torch.Tensor]:
        if len(b) != self.handle.items:
            raise ValueError(f"need {self.handle.items} right-hand sides, got {len(b)}")
        kw = dict(rtol=rtol, atol=atol, max_iter=max_iter, fixed=fixed, jacobi=jacobi)
        return list(_ListSolveFn.apply(self, kw, *self.vals, *b))

    def info(self, backward: bool = False) -> list[dict]:
        buf = self.last_backward_info if backward else self.last_info
        return [] if buf is None else read_info(buf)
