"""ctypes binding of libsla.so (include/sla.h): argument marshalling only.

Every numerical step runs in the HIP kernels behind the C ABI.  Tensors are
passed as raw device pointers with torch's current HIP stream; this module never
computes anything itself and has no CPU fallback: if the library is missing it
raises at import.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsla.so")

SLA_OK, SLA_ERR_INVALID_ARG, SLA_ERR_INVALID_CSR, SLA_ERR_UNSUPPORTED, SLA_ERR_OOM, SLA_ERR_HIP = range(6)
SLA_CONVERGED, SLA_MAX_ITER, SLA_NOT_SPD, SLA_NAN, SLA_BREAKDOWN = range(5)
STATE_NAMES = {0: "CONVERGED", 1: "MAX_ITER", 2: "NOT_SPD", 3: "NAN", 4: "BREAKDOWN"}
SLA_SYMMETRIC = 1
SLA_EAGER_TRANSPOSE = 2
SLA_FIXED_ITERS = 1
SLA_JACOBI = 2
SLA_BICGSTAB = 4
SLA_EIG_LARGEST, SLA_EIG_SMALLEST = 0, 1
SLA_EIG_MAX_K = 32
SLA_EIG_JACOBI = 1
(SLA_K_CG_INIT, SLA_K_CG_SPMV, SLA_K_CG_UPDATE, SLA_K_MATVEC, SLA_K_PATTERN_OUTER,
 SLA_K_GATHER_VALS, SLA_K_TRANSPOSE, SLA_K_CG_PUPD, SLA_K_GROUP_LAYOUT, SLA_K_BS_SPMV, SLA_K_BS_VEC,
 SLA_K_LZ_SPMV, SLA_K_LZ_ORTH, SLA_K_LZ_RITZ, SLA_K_LOB_SPMM, SLA_K_LOB_GRAM, SLA_K_LOB_COMB,
 SLA_K_COUNT) = range(18)
KERNEL_NAMES = ["cg_init", "cg_spmv", "cg_update", "matvec", "pattern_outer", "gather_vals",
                "transpose", "cg_pupd", "group_layout", "bs_spmv", "bs_vec", "lz_spmv", "lz_orth",
                "lz_ritz", "lob_spmm", "lob_gram", "lob_comb"]

EXPORTS = [
    "sla_set_allocator", "sla_csr_create", "sla_csr_destroy", "sla_csr_info", "sla_csr_analysis", "sla_csr_col_bits", "sla_csr_diagonals", "sla_csr_group_window", "sla_matvec", "sla_matvec_backward",
    "sla_solve", "sla_solve_backward", "sla_list_create", "sla_list_destroy", "sla_list_info", "sla_list_col_bits", "sla_list_solve",
    "sla_list_solve_backward", "sla_eigsh", "sla_lobpcg", "sla_eigsh_backward", "sla_timing_enable",
    "sla_timing_reset", "sla_timing_collect", "sla_timing_query", "sla_timing_query_bytes", "sla_status_string",
    "sla_last_error", "sla_version", "sla_probe_stream", "sla_solve_noalloc",
]


class SlaCgOpts(C.Structure):
    _fields_ = [("rtol", C.c_double), ("atol", C.c_double), ("max_iter", C.c_int64),
                ("check_every", C.c_int32), ("flags", C.c_uint32),
                ("residual_history", C.c_void_p)]


class SlaCgInfo(C.Structure):
    _fields_ = [("iterations", C.c_int64), ("res_norm", C.c_double), ("rhs_norm", C.c_double),
                ("state", C.c_int32), ("reserved", C.c_int32)]


assert C.sizeof(SlaCgInfo) == 32


ALLOC_FN = C.CFUNCTYPE(C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p)
FREE_FN = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p, C.c_void_p)


class SlaEigOpts(C.Structure):
    _fields_ = [("tol", C.c_double), ("max_dim", C.c_int64), ("which", C.c_int32),
                ("check_every", C.c_int32), ("max_iter", C.c_int64), ("keep", C.c_int32),
                ("flags", C.c_int32)]


class SlaEigInfo(C.Structure):
    _fields_ = [("iterations", C.c_int64), ("max_res", C.c_double), ("state", C.c_int32),
                ("restarts", C.c_int32)]


class SlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


_lib = None


def _status_name(s: int) -> str:
    return ["SLA_OK", "SLA_ERR_INVALID_ARG", "SLA_ERR_INVALID_CSR", "SLA_ERR_UNSUPPORTED",
            "SLA_ERR_OOM", "SLA_ERR_HIP"][s] if 0 <= s < 6 else f"status {s}"


def load():
    """Load libsla.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python differentiable_sparse_linear_spmv_amd/build.py` "
                          "(there is no CPU fallback)")
    L = C.CDLL(LIB_PATH)
    P, i64, i32, u32 = C.c_void_p, C.c_int64, C.c_int32, C.c_uint32
    st = C.c_int
    L.sla_csr_create.argtypes = [C.POINTER(P), i64, i64, i64, P, i32, P, u32, P]
    L.sla_csr_create.restype = st
    L.sla_csr_destroy.argtypes = [P]
    L.sla_csr_destroy.restype = st
    L.sla_csr_info.argtypes = [P, C.POINTER(i64), C.POINTER(i64), C.POINTER(i64),
                               C.POINTER(i32), C.POINTER(u32), C.POINTER(i64)]
    L.sla_csr_info.restype = st
    L.sla_csr_analysis.argtypes = [P, C.POINTER(i32), C.POINTER(i32), C.POINTER(i32), C.POINTER(i64),
                                   C.POINTER(i32)]
    L.sla_csr_analysis.restype = st
    L.sla_csr_col_bits.argtypes = [P, C.POINTER(i32)]
    L.sla_csr_col_bits.restype = st
    L.sla_csr_diagonals.argtypes = [P, C.POINTER(i32)]
    L.sla_csr_diagonals.restype = st
    L.sla_csr_group_window.argtypes = [P, C.POINTER(i32)]
    L.sla_csr_group_window.restype = st
    L.sla_matvec.argtypes = [P, i64, P, P, P, P]
    L.sla_matvec.restype = st
    L.sla_matvec_backward.argtypes = [P, i64, P, P, P, P, P, P]
    L.sla_matvec_backward.restype = st
    L.sla_solve.argtypes = [P, i64, P, P, P, C.POINTER(SlaCgOpts), P, P]
    L.sla_solve.restype = st
    L.sla_solve_noalloc.argtypes = [P, i64, P, P, P, C.POINTER(SlaCgOpts), P, P]
    L.sla_solve_noalloc.restype = st
    L.sla_solve_backward.argtypes = [P, i64, P, P, P, P, P, C.POINTER(SlaCgOpts), P, P]
    L.sla_solve_backward.restype = st
    L.sla_list_create.argtypes = [C.POINTER(P), i32, P, P, P, i32, P, u32, P]
    L.sla_list_create.restype = st
    L.sla_list_destroy.argtypes = [P]
    L.sla_list_destroy.restype = st
    L.sla_list_info.argtypes = [P, C.POINTER(i64), C.POINTER(i64), C.POINTER(i32)]
    L.sla_list_info.restype = st
    L.sla_list_col_bits.argtypes = [P, C.POINTER(i32)]
    L.sla_list_col_bits.restype = st
    L.sla_list_solve.argtypes = [P, P, P, P, C.POINTER(SlaCgOpts), P, P]
    L.sla_list_solve.restype = st
    L.sla_list_solve_backward.argtypes = [P, P, P, P, P, P, C.POINTER(SlaCgOpts), P, P]
    L.sla_list_solve_backward.restype = st
    L.sla_eigsh.argtypes = [P, P, i32, P, P, P, C.POINTER(SlaEigOpts), C.POINTER(SlaEigInfo), P]
    L.sla_eigsh.restype = st
    L.sla_lobpcg.argtypes = [P, P, i32, P, P, P, C.POINTER(SlaEigOpts), C.POINTER(SlaEigInfo), P]
    L.sla_lobpcg.restype = st
    L.sla_eigsh_backward.argtypes = [P, i32, P, P, P, P]
    L.sla_eigsh_backward.restype = st
    L.sla_set_allocator.argtypes = [ALLOC_FN, FREE_FN, P]
    L.sla_set_allocator.restype = st
    L.sla_timing_enable.argtypes = [i32]
    L.sla_timing_enable.restype = st
    L.sla_timing_reset.argtypes = []
    L.sla_timing_reset.restype = st
    L.sla_timing_collect.argtypes = []
    L.sla_timing_collect.restype = st
    L.sla_timing_query.argtypes = [i32, C.POINTER(i64), C.POINTER(C.c_double)]
    L.sla_timing_query.restype = st
    L.sla_timing_query_bytes.argtypes = [i32, C.POINTER(C.c_double)]
    L.sla_timing_query_bytes.restype = st
    L.sla_probe_stream.argtypes = [i32, i32, P, P, i64, i32, i32, i32, P, P]
    L.sla_probe_stream.restype = st
    L.sla_status_string.argtypes = [st]
    L.sla_status_string.restype = C.c_char_p
    L.sla_last_error.argtypes = []
    L.sla_last_error.restype = C.c_char_p
    L.sla_version.argtypes = []
    L.sla_version.restype = i32
    _lib = L
    return L


def check(status: int) -> None:
    if status != SLA_OK:
        msg = load().sla_last_error().decode(errors="replace")
        raise SlaError(status, msg)
