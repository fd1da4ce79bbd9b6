"""CPU tests of bench.py's host logic: the algorithmic byte models behind the roofline
figures (the per-launch formulas of the kernels, column width included), the basis
positions of a thick-restarted Lanczos run, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench

N, NNZ = 1_048_576, 5_238_784
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("cb", [2, 4])
def test_cg_fused_model(cb):
    m = bench.bytes_model(N, NNZ, 1, 4, col_bytes=cb)
    # values, columns, row pointers; read r, p_{k-1}, x; write p_k, q, x
    assert m["cg_spmv"] == (8 + cb) * NNZ + 4 * (N + 1) + 48 * N
    assert m["cg_update"] == 24 * N                      # read r, q; write r
    assert m["iteration"] == m["cg_spmv"] + m["cg_update"]


def test_cg_split_and_batched_model():
    m = bench.bytes_model(N, NNZ, 8, 4, split=True, col_bytes=2)
    # the pattern is read once per launch, the values and vectors once per system
    assert m["cg_spmv"] == 8 * NNZ * 8 + 2 * NNZ + 4 * (N + 1) + 16 * N * 8
    assert m["cg_pupd"] == 40 * N * 8
    assert m["iteration"] == m["cg_pupd"] + m["cg_spmv"] + m["cg_update"]


def test_column_width_changes_only_the_pattern_term():
    a = bench.bytes_model(N, NNZ, 1, 4, col_bytes=4)
    b = bench.bytes_model(N, NNZ, 1, 4, col_bytes=2)
    assert a["cg_spmv"] - b["cg_spmv"] == 2 * NNZ and a["cg_update"] == b["cg_update"]
    x = bench.bytes_model_bicgstab(N, NNZ, 1, 4, col_bytes=4)
    y = bench.bytes_model_bicgstab(N, NNZ, 1, 4, col_bytes=2)
    assert x["iteration"] - y["iteration"] == 2 * 2 * NNZ   # two products per iteration


def test_bicgstab_model():
    m = bench.bytes_model_bicgstab(N, NNZ, 1, 4, col_bytes=2)
    mat = 10 * NNZ + 4 * (N + 1)
    assert m["iteration"] == (mat + 24 * N) + (mat + 16 * N) + 112 * N


def test_lanczos_positions_and_bytes():
    assert bench.lanczos_positions(5, 0, 0) == [0, 1, 2, 3, 4]
    # a basis of 6 keeping 3: 0..5, then 3..5 after each restart
    assert bench.lanczos_positions(12, 6, 3) == [0, 1, 2, 3, 4, 5, 3, 4, 5, 3, 4, 5]
    n, nnz = 1000, 4960
    e = bench.eigsh_bytes(n, nnz, 4, 40, col_bytes=2)
    fused = sum((3 * j + 14) * 8 * n for j in range(bench.LZ_FUSED_COLS))
    plain = sum((4 * j + 16) * 8 * n for j in range(bench.LZ_FUSED_COLS, 40))
    assert e["lz_orth_total"] == fused + plain
    assert e["lz_spmv"] == 10 * nnz + 4 * (n + 1) + 16 * n


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)


def test_v9_iteration_model():
    # the reported roofline's bytes: 4-byte columns and the stated row-pointer width,
    # whatever the kernels read; nine vector passes per system
    assert bench.bytes_model_v9(N, NNZ, 1, 4) == 12 * NNZ + 4 * (N + 1) + 72 * N
    n, nnz = 169_000_000, 844_948_000
    assert bench.bytes_model_v9(n, nnz, 1, 8) == 12 * nnz + 8 * (n + 1) + 72 * n
    # a batch multiplies the values and vectors, not the pattern
    assert bench.bytes_model_v9(N, NNZ, 4, 4) == 32 * NNZ + 4 * NNZ + 4 * (N + 1) + 288 * N
    # the kernels' own fused model counts the same nine passes
    m = bench.bytes_model(N, NNZ, 1, 4, col_bytes=4)
    assert m["iteration"] == bench.bytes_model_v9(N, NNZ, 1, 4)


def test_host_cpu_report():
    h = bench.host_cpu()
    assert h["nproc"] >= 1 and 1 <= h["threads"] <= h["nproc"]


def test_oracle_timing_mode_follows_the_parity_oracle():
    # the CPU baseline's OpenMP timing mode runs the parity oracle's CG steps: on a
    # small grid its iterates agree with the sequential oracle to rounding
    import numpy as np
    import oracle as O
    import workloads as W
    A = W.poisson5(40)
    b = W.rhs_normal(A.n_rows, 0)
    r = O.cg_timing(A, b, 30, 3)
    f = O.cg(A, b, rtol=0.0, max_iter=30, fixed=True)
    bw = O.solve_backward(A, f["x"], f["x"], rtol=0.0, max_iter=30, fixed=True)
    rel = lambda a, c: np.linalg.norm(a - c) / np.linalg.norm(c)
    assert r["threads"] == 3
    assert rel(r["x"], f["x"]) < 1e-13 and rel(r["lam"], bw["lam"]) < 1e-13
    assert rel(r["gvals"], bw["gvals"]) < 1e-13


def test_diagonal_layout_model():
    # the banded SpMV on the diagonal layout reads nd values per row and a mask, no
    # column indices or row pointers; the vectors and the update are unchanged
    n, nnz = 169_000_000, 844_948_000
    m = bench.bytes_model(n, nnz, 1, 4, col_bytes=2, dia_nd=5)
    assert m["cg_spmv"] == 40 * n + n + 48 * n
    assert m["cg_update"] == 24 * n
    m9 = bench.bytes_model(1000, 8000, 2, 4, dia_nd=9)
    assert m9["cg_spmv"] == 8 * 9 * 1000 * 2 + 2 * 1000 + 48 * 1000 * 2


def test_iteration_roofline_and_resident_ceiling_fields():
    # the bench line's roofline fields from synthetic kernel timings: the V=9 fraction
    # over the whole iteration (SpMV + update), the bytes-moved fraction, and the
    # fraction of same-size streaming probes for a cache-resident workload
    w = dict(name="poisson1024", desc="synthetic", n=N, nnz=NNZ, batch=1, rtol=1e-8, fixed=False, method="cg")
    spmv_ms, upd_ms, launches = 0.022, 0.007, 100
    tq = {"cg_spmv": {"launches": launches, "total_ms": spmv_ms * launches},
          "cg_update": {"launches": launches, "total_ms": upd_ms * launches},
          "cg_pupd": {"launches": 0, "total_ms": 0.0}}
    cr = {"spmv_mix": {"us": 16.0, "gbps": 6500.0}, "triad": {"us": 5.0, "gbps": 5000.0}}
    r = dict(w=w, tq=tq, bicg=False, an={"split": False}, rp_bytes=4, rp_stated=4, col_bytes=2, dia_nd=0,
             spmv_kernel="k_cg_spmv", schedule="fused", steps=1, warmup=0, wall=1.0, event_ms=1.0,
             fwd_it=[1], bwd_it=[1], total_it=2, create_ms=1.0, ceiling_resident=cr)
    assert bench.cache_resident(w)
    roof = bench.cg_summary(r, None, None)["roofline"]
    it_s = spmv_ms * 1e-3 + upd_ms * 1e-3
    v9 = bench.bytes_model_v9(N, NNZ, 1, 4)
    moved = bench.bytes_model(N, NNZ, 1, 4, col_bytes=2)["iteration"]
    assert roof["bytes_per_iteration"] == v9
    assert abs(roof["frac"] - v9 / it_s / 8e12) < 1e-4
    assert abs(roof["frac_bytes_moved"] - moved / it_s / 8e12) < 1e-4
    assert abs(roof["frac_of_resident_ceiling"] - (16.0 + 5.0) / (1e6 * it_s)) < 1e-4
    assert roof["cache_resident"]
    # 169M rows do not fit the Infinity Cache
    assert not bench.cache_resident(dict(w, n=169_000_000, nnz=844_948_000))


def test_oracle_bicgstab_timing_mode_follows_the_parity_oracle():
    # the BiCGStab timing mode runs orc_bicgstab's steps over OpenMP threads, its
    # adjoint on the transpose: on a small nonsymmetric grid the iterates agree with
    # the sequential oracle to rounding
    import numpy as np
    import oracle as O
    import workloads as W
    A = W.convdiff5(30, shift=1.0)
    b = W.rhs_normal(A.n_rows, 0)
    K = 12
    r = O.bicgstab_timing(A, b, K, 3)
    f = O.bicgstab(A, b, rtol=0.0, max_iter=K, fixed=True)
    bw = O.solve_backward(A, f["x"], f["x"], symmetric=False, rtol=0.0, max_iter=K, fixed=True, method="bicgstab")
    rel = lambda a, c: np.linalg.norm(a - c) / np.linalg.norm(c)
    assert r["threads"] == 3
    assert rel(r["x"], f["x"]) < 1e-12 and rel(r["lam"], bw["lam"]) < 1e-12
    assert rel(r["gvals"], bw["gvals"]) < 1e-12
