"""Host-side checks of the C-ABI library (no GPU needed, no compute calls).

* libsla.so loads and exports every function that include/sla.h declares;
* the ctypes structures match the header's layout;
* argument errors are reported before anything touches a device.
"""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sla_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from differentiable_sparse_linear_spmv_amd import _lib
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["sla_csr_create", "sla_csr_destroy", "sla_matvec", "sla_matvec_backward",
                     "sla_solve", "sla_solve_backward"]:
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    from differentiable_sparse_linear_spmv_amd import _lib
    names = declared_functions()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(_lib.EXPORTS) == names


def test_struct_layouts():
    from differentiable_sparse_linear_spmv_amd._lib import SlaCgInfo, SlaCgOpts
    assert C.sizeof(SlaCgInfo) == 32
    assert SlaCgInfo.state.offset == 24
    assert C.sizeof(SlaCgOpts) == 40
    assert SlaCgOpts.residual_history.offset == 32


def test_status_strings_and_version(lib):
    assert lib.sla_status_string(0) == b"SLA_OK"
    assert lib.sla_status_string(2) == b"SLA_ERR_INVALID_CSR"
    assert lib.sla_version() == 100


def test_argument_errors_before_any_device_work(lib):
    from differentiable_sparse_linear_spmv_amd import _lib
    out = C.c_void_p()
    # NULL out pointer
    assert lib.sla_csr_create(None, 4, 4, 0, 1, 32, None, 0, None) == _lib.SLA_ERR_INVALID_ARG
    # bad row pointer width
    assert lib.sla_csr_create(C.byref(out), 4, 4, 0, 1, 16, None, 0, None) == _lib.SLA_ERR_INVALID_ARG
    assert b"row_ptr_bits" in lib.sla_last_error()
    # negative sizes
    assert lib.sla_csr_create(C.byref(out), -1, 4, 0, 1, 32, None, 0, None) == _lib.SLA_ERR_INVALID_ARG
    # too many entries for 32-bit row pointers
    assert lib.sla_csr_create(C.byref(out), 4, 4, 2 ** 31, 1, 32, 1, 0, None) == _lib.SLA_ERR_INVALID_ARG
    # unknown flags, symmetric non-square
    assert lib.sla_csr_create(C.byref(out), 4, 4, 0, 1, 32, None, 64, None) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_csr_create(C.byref(out), 4, 5, 0, 1, 32, None, 1, None) == _lib.SLA_ERR_INVALID_ARG
    # NULL handle on every compute entry point
    assert lib.sla_matvec(None, 1, None, None, None, None) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_matvec_backward(None, 1, None, None, None, None, None, None) == _lib.SLA_ERR_INVALID_ARG
    opts = _lib.SlaCgOpts(1e-8, 0.0, 10, 0, 0, None)
    assert lib.sla_solve(None, 1, None, None, None, C.byref(opts), None, None) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_solve_backward(None, 1, None, None, None, None, None, C.byref(opts), None,
                                  None) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_timing_query(99, None, None) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_csr_destroy(None) == _lib.SLA_OK


def test_package_has_no_cpu_path():
    # The product package must not import the oracle or any CPU solver.
    pkg = os.path.join(ROOT, "differentiable_sparse_linear_spmv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "scipy" not in text and "numpy.linalg" not in text, f


def test_struct_layouts_match_the_compiled_header(tmp_path):
    # sizeof / offsetof from a C program built against include/sla.h, field by field
    import shutil
    import subprocess
    from differentiable_sparse_linear_spmv_amd import _lib
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    structs = {"sla_cg_opts": _lib.SlaCgOpts, "sla_cg_info": _lib.SlaCgInfo, "sla_eig_opts": _lib.SlaEigOpts,
               "sla_eig_info": _lib.SlaEigInfo}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "sla.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["return 0; }"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == C.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_allocator_hook_arguments(lib):
    from differentiable_sparse_linear_spmv_amd import _lib
    assert lib.sla_set_allocator(_lib.ALLOC_FN(), _lib.FREE_FN(), None) == 0     # back to hipMalloc
    only_alloc = _lib.ALLOC_FN(lambda n, s, c: None)
    assert lib.sla_set_allocator(only_alloc, _lib.FREE_FN(), None) == 1         # SLA_ERR_INVALID_ARG
    assert b"both" in lib.sla_last_error()
    assert lib.sla_set_allocator(_lib.ALLOC_FN(), _lib.FREE_FN(), None) == 0
