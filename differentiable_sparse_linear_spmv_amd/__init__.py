"""MI355X-native differentiable sparse linear algebra: CSR SpMV, the
conjugate-gradient solve (plain or Jacobi-preconditioned) and BiCGStab with their
adjoint backward passes, and the Lanczos eigensolver with its Hellmann-Feynman
gradient, as HIP kernels for gfx950 behind a C ABI (include/sla.h, libsla.so).

Importing the package loads libsla.so and fails loudly if it is missing: there
is no CPU path.
"""
from . import _lib
from ._lib import SlaError

_lib.load()

from .sparse import (SparseTensor, SparseTensorList, cg_opts, csr_analysis, csr_create,  # noqa: E402
                     csr_destroy, csr_info, eigsh, eigsh_backward, list_col_bits, list_create, list_solve,
                     list_solve_backward, lobpcg, matvec, matvec_backward, read_info, solve, solve_backward, timing,
                     use_torch_allocator, solve_noalloc, info_buffer)

__all__ = ["SparseTensor", "SparseTensorList", "SlaError", "cg_opts", "csr_analysis", "csr_create", "csr_destroy",
           "csr_info", "eigsh", "eigsh_backward", "list_col_bits", "list_create", "list_solve", "list_solve_backward", "lobpcg",
           "matvec", "matvec_backward", "read_info", "solve", "solve_backward", "timing", "use_torch_allocator",
           "solve_noalloc", "info_buffer"]
