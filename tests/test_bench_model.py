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
