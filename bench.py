#!/usr/bin/env python3
"""Benchmark: fp64 CG iterations/s and achieved HBM bandwidth of the sparse CG
solve + adjoint backward on one MI355X.

One step = one pass of the whole hot path on one batch of synthetic input:
    x = A^{-1} b by conjugate gradients (sla_solve), then the adjoint backward of
    L = 0.5 |x|^2 (sla_solve_backward: A^T lambda = x, dL/db = lambda,
    dL/dA_ij = -lambda_i x_j on the pattern).
The default workload is the 1024 x 1024 5-point Poisson system (n = 1,048,576,
nnz = 5,238,784, b ~ N(0, 1) seed 0, relative residual 1e-8), a stand-in for the
1M-DOF 2-D Poisson benchmark of the torch-sla paper (paperpeel page, section 4.1,
Table 3).  Inputs are resident in HBM before the timed region starts.

--workload convdiff1024 runs BiCGStab (forward, and on A^T in the adjoint) on a
nonsymmetric convection-diffusion system instead; its line reports BiCGStab
iterations per second under its own metric name.

Printed: one JSON line with value = CG iterations per second (forward + adjoint
iterations of all timed steps / wall time), the roofline of the dominant kernel
(algorithmic bytes per launch / HIP-event-timed average launch duration), and the
CPU oracle timed on a bounded sample of the same workload.

Profiling helpers (used to make the summaries under profiles/):
    --calibrate-copy      also run a plain device copy of known size (counter scaling)
    --summarize-pmc DIR   turn rocprofv3 counter CSVs under DIR into a traffic summary
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "fp64 CG iters/s + achieved HBM GB/s, Poisson 1M/169M DOF; solve+adjoint ms"
# the nonsymmetric widening (not the headline metric): BiCGStab on convection-diffusion
METRIC_LIST = "fp64 CG iters/s summed over items + achieved HBM GB/s, SparseTensorList of 64 Poisson grids; solve+adjoint ms"
METRIC_EIGSH = "fp64 Lanczos steps/s + achieved HBM GB/s, eigsh on a 1M-DOF Poisson-type matrix; eigsh+gradient ms"
METRIC_LOBPCG = "fp64 LOBPCG iterations/s + achieved HBM GB/s, eigsh on a 1M-DOF Poisson-type matrix; eigsh+gradient ms"
LOBPCG_FAMILIES = {"lob_spmm": ["k_blk_spmm"], "lob_gram": ["k_blk_gram", "k_blk_reduce"], "lob_comb": ["k_blk_comb"]}
METRIC_BICGSTAB = "fp64 BiCGStab iters/s + achieved HBM GB/s, convection-diffusion 1M DOF; solve+adjoint ms"
COPY_BYTES = 1 << 30            # calibration copy: 1 GiB read + 1 GiB written


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "differentiable_sparse_linear_spmv_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------------------ bytes model
def bytes_model(n: int, nnz: int, batch: int, rp_bytes: int, split: bool = False, col_bytes: int = 4,
                dia_nd: int = 0) -> dict:
    """Algorithmic HBM bytes of the kernels, per launch (all systems of the batch).

    rp_bytes is the width of the row pointers the kernels read: 4 whenever nnz < 2^31
    (the library keeps a 32-bit copy of 64-bit row pointers that fit).  col_bytes is
    the width of the column indices the SpMV reads: 2 where the handle holds 16-bit
    column offsets (sla_csr_col_bits), else 4.  dia_nd > 0: the banded SpMV reads the
    diagonal layout instead of the CSR arrays: dia_nd values per row and system (absent
    entries' slots included) and a mask of 1 byte per row (2 above 8 diagonals), no
    column indices and no row pointers.

    Fused schedule (plain or banded SpMV):
      cg_spmv  : values 8 nnz B + columns col_bytes nnz + row pointers rp (n + 1)
                 + vectors: read r, p_{k-1}, x; write p_k, q, x   -> 6 x 8 n B
      cg_update: read r, q; write r                              -> 3 x 8 n B
      one CG iteration = both (nine vector passes).
    Split schedule (unstructured patterns):
      cg_pupd  : read r, p_{k-1}, x; write p_k, x                 -> 5 x 8 n B
      cg_spmv  : values, columns, row pointers + read p_k (own row; the gathers are
                 cache traffic), write q                          -> 2 x 8 n B
      cg_update: as above; one iteration = ten vector passes.
    """
    if dia_nd > 0:
        mat = 8 * dia_nd * n * batch + (1 if dia_nd <= 8 else 2) * n
    else:
        mat = 8 * nnz * batch + col_bytes * nnz + rp_bytes * (n + 1)
    upd = 3 * 8 * n * batch
    if split:
        pupd = 5 * 8 * n * batch
        spmv = mat + 2 * 8 * n * batch
        return dict(cg_pupd=pupd, cg_spmv=spmv, cg_update=upd, iteration=pupd + spmv + upd,
                    flops_iteration=(2 * nnz + 10 * n) * batch)
    spmv = mat + 6 * 8 * n * batch
    return dict(cg_spmv=spmv, cg_update=upd, iteration=spmv + upd,
                flops_iteration=(2 * nnz + 10 * n) * batch)


def bytes_model_v9(n: int, nnz: int, batch: int, rp_stated: int) -> int:
    """Bytes of one CG iteration in the reported roofline model: values 8 nnz per
    system, 4-byte column indices and row pointers of the width the workload states
    (read once per iteration, shared by the batch), and nine passes over n-vectors
    per system (read r, p_{k-1}, x and write p_k, q, x around the SpMV; read r, q and
    write r in the update: the fewest a Hestenes-Stiefel iteration with a stored q
    needs).  The fraction against it moves only with the iteration's time."""
    return 8 * nnz * batch + 4 * nnz + rp_stated * (n + 1) + 72 * n * batch


def bytes_model_bicgstab(n: int, nnz: int, batch: int, rp_bytes: int, col_bytes: int = 4) -> dict:
    """Algorithmic HBM bytes of the BiCGStab kernels, per launch (all systems).

      v = A p  : values, columns, row pointers + read p (the gathers are cache traffic)
                 and rh, write v                                    -> 3 x 8 n B
      t = A s  : values, columns, row pointers + read s, write t    -> 2 x 8 n B
      bs_spmv  : the mean of the two (the timing id covers both launches)
      p update : read r, p, v; write p -> 4;  s: read r, v; write s -> 3;
      update   : read x, p, s, t, rh; write x, r -> 7;  bs_vec: the mean of the three
      one iteration = both products + 14 vector passes.
    """
    mat = 8 * nnz * batch + col_bytes * nnz + rp_bytes * (n + 1)
    v = 8 * n * batch
    spmv_v, spmv_t = mat + 3 * v, mat + 2 * v
    vec = 14 * v
    return dict(bs_spmv=(spmv_v + spmv_t) / 2, bs_vec=vec / 3, iteration=spmv_v + spmv_t + vec,
                flops_iteration=(4 * nnz + 24 * n) * batch)


LZ_FUSED_COLS = 32   # the library's fused update-and-dots threshold (bases of <= 32 vectors)


def lanczos_positions(steps: int, max_dim: int, keep: int) -> list:
    """Basis position j of every Lanczos step: 0 .. max_dim - 1, then after each thick
    restart keep .. max_dim - 1 again (no restart: 0 .. steps - 1)."""
    if max_dim <= 0 or steps <= max_dim:
        return list(range(steps))
    pos, left = list(range(max_dim)), steps - max_dim
    while left > 0:
        c = min(left, max_dim - keep)
        pos += list(range(keep, keep + c))
        left -= c
    return pos


def eigsh_bytes(n: int, nnz: int, rp_bytes: int, steps: int, max_dim: int = 0, keep: int = 0,
                restarts: int = 0, col_bytes: int = 4) -> dict:
    """Algorithmic HBM bytes of a Lanczos run of `steps` steps.

      lz_spmv  (per step): values, columns, row pointers + read v_j (the gathers are
               cache traffic), write w                              -> mat + 2 x 8 n
      lz_orth  (step at basis position j): three-term step (read v_j, v_{j-1}, w; write
               w) 4 x 8 n; two Gram-Schmidt passes, each: dots read V_{0..j} and w,
               (j + 2) x 8 n, update read V_{0..j} and w, write w, (j + 3) x 8 n; next
               vector (read w, write v_{j+1}) 2 x 8 n               -> (4 j + 16) x 8 n
               with j + 1 <= LZ_FUSED_COLS the first update and the second dots
               share one read of V and w (and one write of w)       -> (3 j + 14) x 8 n
               plus, on the first step after a restart, the couplings: read V_{0..keep-1}
               and w, write w                                       -> (keep + 2) x 8 n
      restart  (per restart, timed with the Ritz kernels): read V_{0..m-1}, write
               V_{0..keep-1}, copy v_m                               -> (m + keep + 2) x 8 n
      lz_ritz  u_r = V s_r: read V_{0..m-1} once, write k vectors (plus the start)
    """
    mat = 8 * nnz + col_bytes * nnz + rp_bytes * (n + 1)
    spmv = mat + 2 * 8 * n
    pos = lanczos_positions(steps, max_dim, keep)
    orth = sum(((3 * j + 14) if j + 1 <= LZ_FUSED_COLS else (4 * j + 16)) * 8 * n for j in pos) \
        + restarts * (keep + 2) * 8 * n
    rst = restarts * (max_dim + keep + 2) * 8 * n
    return dict(lz_spmv=spmv, lz_orth_total=orth, restart_total=rst, run=steps * spmv + orth + rst)


def run_eigsh(args, w, S, torch) -> dict:
    """One step = eigsh (k wanted pairs) + the gradient of sum(lambda)."""
    h = S.csr_create(w["rp"], w["col"], symmetric=True)
    vals, v0, k = w["vals"], w["v0"], w["k"]

    def step():
        ev, U, info = S.eigsh(h, vals, k, v0, which=w["which"], tol=w["tol"], max_dim=w["max_dim"],
                              max_iter=w["max_iter"], keep=w["keep"])
        gv = S.eigsh_backward(h, U, torch.ones(k, dtype=torch.float64, device=vals.device))
        return ev, U, gv, info

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    infos = [step()[3] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    steps_run = infos[-1]["iterations"]
    # per-kernel HIP-event timing of one more run
    S.timing.reset()
    S.timing.enable(True)
    step()
    S.timing.collect()
    S.timing.enable(False)
    tq = S.timing.query()
    n, nnz = w["n"], w["nnz"]
    keep = w["keep"] or min(w["max_dim"] - 1, max(k + 1, (w["max_dim"] + k) // 2))
    bm = eigsh_bytes(n, nnz, 4, steps_run, w["max_dim"], keep, infos[-1]["restarts"],
                     col_bytes=S.csr_analysis(h)["col_bits"] // 8)
    orth_ms = tq["lz_orth"]["total_ms"]
    spmv_ms = tq["lz_spmv"]["total_ms"] / max(tq["lz_spmv"]["launches"], 1)
    achieved = bm["lz_orth_total"] / (orth_ms * 1e-3) / 1e9
    return dict(value=sum(i["iterations"] for i in infos) / wall, wall=wall, tq=tq, bm=bm, achieved=achieved,
                spmv_ms=spmv_ms, orth_ms=orth_ms, info=infos[-1],
                spmv_gbps=bm["lz_spmv"] / (spmv_ms * 1e-3) / 1e9)


def run_lobpcg(args, c, S, torch, dev) -> dict:
    """One step = LOBPCG (k wanted pairs) + the gradient of sum(lambda).  The roofline
    kernel is the block-kernel family with the most time; its algorithmic bytes are
    counted by the library per launch (each operand column read once, each output
    written once, the matrix once per product)."""
    A = c["A"]
    h = S.csr_create(torch.from_numpy(A.row_ptr).to(dev), torch.from_numpy(A.col).to(dev), symmetric=True)
    vals = torch.from_numpy(A.vals).to(dev)
    X0 = torch.from_numpy(c["X0"]).to(dev)
    k = c["k"]

    def step():
        ev, U, info = S.lobpcg(h, vals, k, X0, which=c["which"], tol=c["tol"], max_iter=c["max_iter"])
        S.eigsh_backward(h, U, torch.ones(k, dtype=torch.float64, device=dev))
        return info

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    infos = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    S.timing.reset()
    S.timing.enable(True)
    step()
    S.timing.collect()
    S.timing.enable(False)
    tq = S.timing.query()
    fam = max(LOBPCG_FAMILIES, key=lambda f: tq[f]["total_ms"])
    achieved = tq[fam]["bytes"] / (tq[fam]["total_ms"] * 1e-3) / 1e9
    return dict(value=sum(i["iterations"] for i in infos) / wall, wall=wall, tq=tq, info=infos[-1], fam=fam,
                achieved=achieved)


def cpu_baseline_lobpcg(c, iters: int) -> dict:
    """The oracle's LOBPCG for a bounded number of iterations: with its library calls on
    every host thread (the value), and on one thread beside it."""
    import oracle.lobpcg as OL
    from threadpoolctl import threadpool_limits
    host = host_cpu()
    out = {}
    for nt in (host["threads"], 1):
        t0 = time.perf_counter()
        with threadpool_limits(nt):
            OL.lobpcg(c["A"], c["k"], c["X0"], which=c["which"], tol=1e-300, max_iter=iters)
        dt = time.perf_counter() - t0
        out[nt] = dict(value=round(iters / dt, 3), unit="LOBPCG iterations/s", cores=nt, kind="oracle",
                       sample=f"oracle LOBPCG on this workload, the first {iters} iterations, its numpy "
                              f"calls on {nt} thread(s)", seconds=round(dt, 2))
    r = dict(out[host["threads"]], nproc=host["nproc"], host_model=host["model"])
    if host["threads"] != 1:
        r["single_thread"] = out[1]
    return r


def run_list(args, c, S, torch, dev) -> dict:
    """One step = sla_list_solve + sla_list_solve_backward over every item."""
    import numpy as np
    items = c["items"]
    h = S.list_create([torch.from_numpy(A.row_ptr).to(dev) for A in items],
                      [torch.from_numpy(A.col).to(dev) for A in items], symmetric=True)
    vals = [torch.from_numpy(A.vals).to(dev) for A in items]
    bs = [torch.from_numpy(b).to(dev) for b in c["b"]]
    opts = S.cg_opts(rtol=c["rtol"], max_iter=c["max_iter"])

    def step():
        x, info = S.list_solve(h, vals, bs, opts)
        gb, gv, binfo = S.list_solve_backward(h, vals, x, [xi.clone() for xi in x], opts)
        return info, binfo

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    infos = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fi = [s["iterations"] for s in S.read_info(infos[-1][0])]
    bi = [s["iterations"] for s in S.read_info(infos[-1][1])]
    S.timing.reset()
    S.timing.enable(True)
    step()
    S.timing.collect()
    S.timing.enable(False)
    tq = S.timing.query()
    # algorithmic bytes of every item-iteration of the fused CG SpMV, over its measured time
    cb = S.list_col_bits(h) // 8
    per_item = [bytes_model(A.n_rows, A.nnz, 1, 4, col_bytes=cb)["cg_spmv"] for A in items]
    spmv_bytes = float(np.dot(np.array(fi) + np.array(bi), per_item))
    it_bytes = float(np.dot(np.array(fi) + np.array(bi), [bytes_model(A.n_rows, A.nnz, 1, 4, col_bytes=cb)["iteration"]
                                                          for A in items]))
    spmv_ms = tq["cg_spmv"]["total_ms"]
    iter_ms = spmv_ms + tq["cg_update"]["total_ms"] + tq["cg_pupd"]["total_ms"]
    return dict(value=(sum(fi) + sum(bi)) * args.steps / wall, wall=wall, tq=tq, fi=fi, bi=bi,
                achieved=spmv_bytes / (spmv_ms * 1e-3) / 1e9, spmv_bytes=spmv_bytes, spmv_ms=spmv_ms,
                iter_gbps=it_bytes / (iter_ms * 1e-3) / 1e9, info=S.list_info if hasattr(S, "list_info") else None)


def cpu_baseline_list(c, iters: int) -> dict:
    """The oracle on every item of the list, a fixed number of iterations each.

    The value: the oracle's timing mode over items, one host thread per item at a time
    (each the CG steps on one OpenMP thread; the C calls release Python's lock), on all
    host threads.  Beside it, the parity oracle on one thread."""
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor
    host = host_cpu()
    k = len(c["items"])
    t0 = time.perf_counter()
    for A, b in zip(c["items"], c["b"]):
        f = O.cg(A, b, rtol=0.0, max_iter=iters, fixed=True)
        O.solve_backward(A, f["x"], f["x"], symmetric=True, rtol=0.0, max_iter=iters, fixed=True)
    dt1 = time.perf_counter() - t0
    single = dict(value=round(2 * iters * k / dt1, 3), unit="CG iters/s (summed over items)", cores=1,
                  kind="oracle", sample=f"parity mode (sequential oracle) on each of the {k} items, {iters} fixed "
                                        f"iterations + {iters} adjoint", seconds=round(dt1, 2))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=host["threads"]) as ex:
        list(ex.map(lambda ab: O.cg_timing(ab[0], ab[1], iters, 1, adjoint=True), zip(c["items"], c["b"])))
    dt = time.perf_counter() - t0
    return dict(value=round(2 * iters * k / dt, 3), unit="CG iters/s (summed over items)", cores=host["threads"],
                kind="oracle", mode="timing mode over items: one host thread per item, each the oracle's CG steps "
                                    "on one OpenMP thread",
                sample=f"oracle CG on each of the {k} items, {iters} fixed iterations + {iters} adjoint, "
                       f"{host['threads']} items at once", seconds=round(dt, 2), nproc=host["nproc"],
                host_model=host["model"], single_thread=single)


def cpu_baseline_eigsh(w, steps: int) -> dict:
    """The oracle's Lanczos for a bounded number of steps of the same problem: with its
    library calls on every host thread (the value), and on one thread beside it."""
    import oracle.eigsh as OE
    from threadpoolctl import threadpool_limits
    A = w["host"]["A"]
    host = host_cpu()
    out = {}
    for nt in (host["threads"], 1):
        t0 = time.perf_counter()
        with threadpool_limits(nt):
            if w["max_dim"] and w["max_dim"] < steps:
                OE.eigsh(A, w["k"], w["host"]["v0"], which=w["which"], tol=1e-300, max_dim=w["max_dim"],
                         max_iter=steps, keep=w["keep"] or None)
                how = f"step budget, basis of {w['max_dim']} with thick restart"
            else:
                OE.eigsh(A, w["k"], w["host"]["v0"], which=w["which"], tol=1e-300, max_dim=steps)
                how = "dimension cap"
        dt = time.perf_counter() - t0
        out[nt] = dict(value=round(steps / dt, 3), unit="Lanczos steps/s", cores=nt, kind="oracle",
                       sample=f"oracle Lanczos on this workload, the first {steps} steps ({how}), its numpy "
                              f"calls on {nt} thread(s)", seconds=round(dt, 2))
    r = dict(out[host["threads"]], nproc=host["nproc"], host_model=host["model"])
    if host["threads"] != 1:
        r["single_thread"] = out[1]
    return r


# ------------------------------------------------------------------------------ workloads
def make_workload(name: str, device):
    import numpy as np
    import torch
    import workloads as W

    if name == "poisson13000":
        c = W.config(name)
        N = c["N"]
        rp, col, vals = W.poisson5_torch(N, device, index64=True)
        b = torch.from_numpy(W.rhs_normal(N * N, 0)).to(device)
        return dict(name=name, n=N * N, nnz=col.numel(), batch=1, rp=rp, col=col, vals=vals, b=b,
                    rtol=0.0, max_iter=c["max_iter"], fixed=True, loss="half_sq", host=None,
                    method="cg", symmetric=True,
                    desc=f"5-point Poisson {N}x{N}, int64 row_ptr handed in (the kernels read an int32 copy: "
                         f"nnz < 2^31), b~N(0,1) seed 0, "
                         f"{c['max_iter']} fixed CG iterations + {c['max_iter']} adjoint")
    c = W.config(name)
    A = c["A"]
    if c.get("method") == "eigsh":
        return dict(name=name, n=A.n_rows, nnz=A.nnz, batch=1, rp=torch.from_numpy(A.row_ptr).to(device),
                    col=torch.from_numpy(A.col).to(device), vals=torch.from_numpy(A.vals).to(device),
                    v0=torch.from_numpy(c["v0"]).to(device), k=c["k"], which=c["which"], tol=c["tol"],
                    max_dim=c["max_dim"], max_iter=c["max_iter"], keep=c["keep"],
                    method="eigsh", host=c,
                    desc=f"Lanczos eigsh: {c['k']} {c['which']} eigenpairs of the variable-coefficient "
                         f"Poisson matrix 1024x1024 (kappa=exp(GRF) seed 0), tol {c['tol']}, v0~N(0,1) "
                         f"seed 3, + Hellmann-Feynman gradient of sum(lambda)"
                         + (f"; thick restart, basis {c['max_dim']}" if c["max_iter"] > c["max_dim"] else ""))
    B = A.batch
    vals = torch.from_numpy(np.ascontiguousarray(A.vals.reshape(B, A.nnz) if B > 1 else A.vals))
    b = torch.from_numpy(np.ascontiguousarray(c["b"]))
    out = dict(name=name, n=A.n_rows, nnz=A.nnz, batch=B,
               rp=torch.from_numpy(A.row_ptr).to(device), col=torch.from_numpy(A.col).to(device),
               vals=vals.to(device), b=b.to(device), rtol=c["rtol"], max_iter=c["max_iter"],
               fixed=False, loss=c["loss"], host=c)
    out["x_target"] = (torch.from_numpy(c["x_target"]).to(device) if "x_target" in c else None)
    descs = {
        "poisson64": "5-point Poisson 64x64 (n=4096), b~U[-1,1] seed 0, CG to 1e-10 + adjoint",
        "poisson1024": "5-point Poisson 1024x1024 (n=1048576, nnz=5238784), b~N(0,1) seed 0, "
                       "CG to 1e-8 + adjoint of 0.5|x|^2",
        "varcoef2048": "variable-coefficient Poisson 2048x2048, kappa=exp(GRF), CG to 1e-8 + adjoint",
        "fem256x256": "256 P1 FEM systems on a jittered 256x256-vertex mesh, CG to 1e-8 + adjoint",
        "graph1m": "graph Laplacian + I of a power-law graph (2^20 nodes, average degree 8, exponent 2.5, "
                   "random node order, seed 0): skewed row lengths, CG to 1e-8 + adjoint of 0.5|x|^2",
        "convdiff1024": "nonsymmetric convection-diffusion 1024x1024 (upwind, recirculating wind W=100), "
                        "b~N(0,1) seed 0, BiCGStab to 1e-8 + BiCGStab adjoint on A^T",
    }
    out["method"] = c.get("method", "cg")
    out["symmetric"] = c.get("symmetric", True)
    out["desc"] = descs[name]
    return out


def loss_grad(w, x):
    if w["loss"] == "sq_target":
        return 2.0 * (x - w["x_target"])
    return x.clone()


# ------------------------------------------------------------------------------ CPU baseline
def host_cpu() -> dict:
    """The host the CPU baseline runs on: CPU model, cores this process may use, and
    the OpenMP threads the timing mode takes (OMP_NUM_THREADS caps them when set)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(nproc, int(omp)) if omp.isdigit() and int(omp) > 0 else nproc
    return dict(model=model, nproc=nproc, threads=threads)


def cpu_baseline(w, iters: int, single_iters: int = 100) -> dict:
    """The oracle timed on this host's cores, on a bounded sample of the workload.

    Timing mode (the value): the oracle's CG steps with its SpMV rows, vector updates
    and inner products split over OpenMP threads (orc_cg_timing), `iters` fixed
    iterations forward and `iters` in the adjoint.  Parity mode beside it: the
    single-threaded oracle itself (orc_cg + orc_solve_backward), `single_iters` + `single_iters`.
    BiCGStab workloads: orc_bicgstab_timing (the adjoint on the transpose), parity mode beside it."""
    import oracle as O
    import workloads as W

    host = host_cpu()
    if w["host"] is None:      # the 169M case: sample a 2048 x 2048 grid of the same stencil
        A = W.poisson5(2048)
        b = W.rhs_normal(A.n_rows, 0)
        vals = None
        what = "the same 5-point stencil at 2048x2048 (169M rows do not fit a bounded CPU sample)"
    else:
        A = w["host"]["A"]
        b = w["host"]["b"].reshape(A.batch, A.n_rows)[0]
        vals = A.vals.reshape(A.batch, A.nnz)[0]
        what = "system 0 of this workload"
    method = w.get("method", "cg")
    unit = "BiCGStab iters/s" if method == "bicgstab" else "CG iters/s"
    name = "BiCGStab" if method == "bicgstab" else "CG"

    si = single_iters if method == "cg" else iters
    t0 = time.perf_counter()
    f = O.cg(A, b, rtol=0.0, max_iter=si, fixed=True, vals=vals, method=method)
    O.solve_backward(A, f["x"], f["x"], symmetric=w.get("symmetric", True), rtol=0.0, max_iter=si,
                     fixed=True, vals=vals, method=method)
    dt1 = time.perf_counter() - t0
    single = dict(value=round(2 * si / dt1, 3), unit=unit, cores=1, kind="oracle",
                  sample=f"parity mode (sequential oracle) on {what}, {si} fixed iterations + {si} adjoint",
                  seconds=round(dt1, 2))
    if method == "bicgstab":
        # the BiCGStab timing mode: orc_bicgstab's steps over OpenMP threads, the adjoint
        # on the transpose
        t0 = time.perf_counter()
        r = O.bicgstab_timing(A, b, iters, host["threads"], adjoint=True, vals=vals)
        dt = time.perf_counter() - t0
        return dict(value=round(2 * iters / dt, 3), unit=unit, cores=r["threads"], kind="oracle",
                    mode="timing mode: the oracle's BiCGStab steps with OpenMP over rows (and over the inner "
                         "products' slices), the adjoint on the transpose",
                    sample=f"oracle {name} on {what}, {iters} fixed iterations + {iters} adjoint iterations "
                           f"on {r['threads']} threads", seconds=round(dt, 2),
                    nproc=host["nproc"], host_model=host["model"], single_thread=single)
    if method != "cg" or not w.get("symmetric", True):
        single.update(nproc=host["nproc"], host_model=host["model"])
        return single
    t0 = time.perf_counter()
    r = O.cg_timing(A, b, iters, host["threads"], adjoint=True, vals=vals)
    dt = time.perf_counter() - t0
    rows = dict(value=round(2 * iters / dt, 3), unit=unit, cores=r["threads"], kind="oracle",
                mode="timing mode: the oracle's CG steps with OpenMP over rows (and over the inner "
                     "products' slices)",
                sample=f"oracle {name} on {what}, {iters} fixed iterations + {iters} adjoint iterations "
                       f"on {r['threads']} threads", seconds=round(dt, 2),
                nproc=host["nproc"], host_model=host["model"], single_thread=single)
    if w["host"] is None or A.batch == 1:
        return rows
    # A batch of systems: the timing mode over systems, one host thread per system (each
    # runs the oracle's CG steps on one OpenMP thread; the C calls release the GIL), on
    # as many systems as there are threads; iterations summed over the systems.
    from concurrent.futures import ThreadPoolExecutor
    nsys = min(host["threads"], A.batch)
    bs = w["host"]["b"].reshape(A.batch, A.n_rows)
    vs = A.vals.reshape(A.batch, A.nnz)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=nsys) as ex:
        list(ex.map(lambda s_: O.cg_timing(A, bs[s_], iters, 1, adjoint=True, vals=vs[s_]), range(nsys)))
    dt = time.perf_counter() - t0
    return dict(value=round(2 * iters * nsys / dt, 3), unit=unit + " (summed over systems)", cores=nsys,
                kind="oracle",
                mode="timing mode over systems: one thread per system, each the oracle's CG steps on one "
                     "OpenMP thread",
                sample=f"oracle {name} on systems 0..{nsys - 1} of this workload, {iters} fixed iterations "
                       f"+ {iters} adjoint iterations each, {nsys} systems at once", seconds=round(dt, 2),
                nproc=host["nproc"], host_model=host["model"], rows_parallel=rows, single_thread=single)


# ------------------------------------------------------------------------------ traffic
def traffic_file(workload: str) -> str:
    kind = "lz_orth" if workload.startswith("eigsh") else "blk" if workload.startswith("lobpcg") else "cg_spmv"
    return os.path.join(ROOT, "profiles", f"{kind}_{workload}_traffic.txt")


def read_traffic(workload: str, key: str = "bytes_per_launch"):
    p = traffic_file(workload)
    if not os.path.exists(p):
        return None, "no counter summary"
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    if key == "bytes_per_iteration" and key not in t:
        parts = [t.get("bytes_per_launch"), t.get("update_bytes_per_launch")]
        if None in parts:
            return None, "no counter summary of every kernel of the iteration"
        return sum(parts) + (t.get("pupd_bytes_per_launch") or 0.0), \
            "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated (SpMV + update + p update launches)"
    return t.get(key), "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated"


def calibrate_copy(torch, dev) -> None:
    """Three plain device copies of COPY_BYTES (the counters' scale), after the run."""
    src = torch.empty(COPY_BYTES // 8, dtype=torch.float64, device=dev).normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str) -> None:
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by the calibration copy.

    Per kernel, the median over its dispatches (a fixed-iteration run: every dispatch
    but the final stop one does the same work).  The copy is the last three
    __amd_rocclr_copyBuffer dispatches: the --calibrate-copy device copies of 1 GiB
    (run after everything else).
    """
    import csv
    import statistics

    def load(d, counter):
        rows = []
        for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(p) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return sorted(rows)

    def per_kernel(rows, key):
        v = [val for _, name, val in rows if key in name]
        return (statistics.median(v), len(v)) if v else (None, 0)

    def copy_of(rows):
        # the calibration copies are the last three device copies of the run
        v = [val for _, name, val in rows if "copyBuffer" in name][-3:]
        return statistics.median(v) if v else None

    fr, wr = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy_f, copy_w = copy_of(fr), copy_of(wr)
    def pick(rows, names):
        for nm in names:
            v = per_kernel(rows, nm)
            if v[0] is not None:
                return v
        return None, 0

    kib = 1024.0
    sf = COPY_BYTES / (copy_f * kib) if copy_f else 1.0
    sw = COPY_BYTES / (copy_w * kib) if copy_w else 1.0
    if workload.startswith("lobpcg"):
        # per family of block kernels, the sum over one run's dispatches (one gradient
        # kernel per run counts the runs)
        runs = sum(1 for _, name, _ in fr if "k_eig_grad" in name)
        runs_w = sum(1 for _, name, _ in wr if "k_eig_grad" in name)
        fams = {}
        for fam, names in LOBPCG_FAMILIES.items():
            tf = sum(val for _, name, val in fr if any(nm in name for nm in names))
            tw = sum(val for _, name, val in wr if any(nm in name for nm in names))
            fams[fam] = dict(kernels=names, fetch_kib_total=tf, write_kib_total=tw,
                             bytes_per_run=(tf * kib * sf / runs + tw * kib * sw / runs_w) if runs and runs_w else None)
        cmd = ("rocprofv3 --pmc {FETCH_SIZE|WRITE_SIZE} -d <dir> -o p --output-format csv -- "
               f"python3 -u bench.py --workload {workload} --steps 1 --warmup 0 --no-cpu-baseline --no-ceiling "
               "--calibrate-copy; then python bench.py --workload "
               f"{workload} --summarize-pmc <fetch dir> <write dir>")
        out = dict(workload=workload, command=cmd, kernel_source_hash=kernel_source_hash(), unit="run",
                   runs=[runs, runs_w], copy_fetch_kib=copy_f, copy_write_kib=copy_w, fetch_scale=sf,
                   write_scale=sw, families=fams)
        with open(traffic_file(workload), "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out))
        return
    if workload.startswith("eigsh") or workload == "poisson_list64":
        # whole runs: the sum over the dispatches of the roofline's kernels, divided by
        # the runs (a kernel launched a known number of times per run counts them)
        if workload.startswith("eigsh"):
            names, per, unit = ["k_lz_three", "k_lz_dots", "k_lz_reduce", "k_lz_axpy", "k_lz_next"], \
                ("k_lz_norm", 1), "run"
        else:
            names, per, unit = ["k_cg_spmv"], ("k_cg_init", 2), "step"

        def total(rows):
            return sum(val for _, name, val in rows if any(nm in name for nm in names))

        runs = sum(1 for _, name, _ in fr if per[0] in name) / per[1]
        runs_w = sum(1 for _, name, _ in wr if per[0] in name) / per[1]
        tf, tw = total(fr), total(wr)
        cmd = ("rocprofv3 --pmc {FETCH_SIZE|WRITE_SIZE} -d <dir> -o p --output-format csv -- "
               f"python3 -u bench.py --workload {workload} --steps 1 --warmup 0 --no-cpu-baseline --no-ceiling "
               "--calibrate-copy; then python bench.py --workload "
               f"{workload} --summarize-pmc <fetch dir> <write dir>")
        out = dict(workload=workload, command=cmd, kernel_source_hash=kernel_source_hash(), kernels=names,
                   unit=unit, runs=[runs, runs_w], fetch_kib_total=tf, write_kib_total=tw,
                   copy_fetch_kib=copy_f, copy_write_kib=copy_w, fetch_scale=sf, write_scale=sw,
                   **{f"bytes_per_{unit}": (tf * kib * sf / runs + tw * kib * sw / runs_w)
                      if runs and runs_w else None})
        p = traffic_file(workload)
        with open(p, "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out))
        return

    spmv_f, nf = pick(fr, ["k_cg_spmv", "k_gcg_spmv"])
    spmv_w, nw = pick(wr, ["k_cg_spmv", "k_gcg_spmv"])
    upd_f, _ = pick(fr, ["k_cg_update", "k_gcg_update"])
    upd_w, _ = pick(wr, ["k_cg_update", "k_gcg_update"])
    pupd_f, _ = pick(fr, ["k_cg_pupd", "k_gcg_pupd", "k_bs_pupd"])
    pupd_w, _ = pick(wr, ["k_cg_pupd", "k_gcg_pupd", "k_bs_pupd"])
    if upd_f is None:   # BiCGStab
        upd_f, _ = pick(fr, ["k_bs_update"])
        upd_w, _ = pick(wr, ["k_bs_update"])
    cmd = ("rocprofv3 --pmc {FETCH_SIZE|WRITE_SIZE} -d <dir> -o p --output-format csv -- "
           f"python3 -u bench.py --workload {workload} --steps 1 --warmup 0 --no-cpu-baseline --no-ceiling "
           "--calibrate-copy --fixed-iters 12; then python bench.py --workload "
           f"{workload} --summarize-pmc <fetch dir> <write dir>")
    out = dict(workload=workload, command=cmd, kernel_source_hash=kernel_source_hash(),
               fetch_kib_per_launch=spmv_f, write_kib_per_launch=spmv_w, launches=[nf, nw],
               copy_fetch_kib=copy_f, copy_write_kib=copy_w, fetch_scale=sf, write_scale=sw,
               bytes_per_launch=(spmv_f * kib * sf + spmv_w * kib * sw) if spmv_f and spmv_w else None,
               update_bytes_per_launch=(upd_f * kib * sf + upd_w * kib * sw) if upd_f and upd_w else None,
               pupd_bytes_per_launch=(pupd_f * kib * sf + pupd_w * kib * sw) if pupd_f and pupd_w else None)
    p = traffic_file(workload)
    with open(p, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


# ------------------------------------------------------------------------------ main
def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="poisson1024",
                    choices=["poisson64", "poisson1024", "varcoef2048", "fem256x256", "poisson13000", "graph1m",
                             "convdiff1024", "eigsh_varcoef1024", "eigsh_tr_varcoef1024", "lobpcg_varcoef1024",
                             "poisson_list64"])
    ap.add_argument("--cpu-iters", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--jacobi", action="store_true",
                    help="Jacobi-preconditioned CG (SLA_JACOBI) instead of the plain CG of the metric")
    ap.add_argument("--fixed-iters", type=int, default=0,
                    help="profiling runs: exactly this many CG iterations per solve")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--no-big", action="store_true",
                    help="skip the 169M-DOF leg of the default poisson1024 line")
    ap.add_argument("--big-steps", type=int, default=3,
                    help="timed steps of the 169M-DOF leg (500 + 500 fixed iterations each)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-bandwidth ceiling")
    ap.add_argument("--ceiling-sweep", action="store_true",
                    help="only run the streaming probes (every variant) and print the best of each mix")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        return 2
    rank = int(os.environ.get("RANK", "0"))

    import torch
    import differentiable_sparse_linear_spmv_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "lobpcg_varcoef1024":
        import workloads as W
        c = W.config(args.workload)
        r = run_lobpcg(args, c, S, torch, dev)
        if args.calibrate_copy:
            calibrate_copy(torch, dev)
        traffic, traffic_src = None, "no counter summary"
        p = traffic_file(args.workload)
        if os.path.exists(p):
            with open(p) as f:
                t = json.load(f)
            if t.get("kernel_source_hash") != kernel_source_hash():
                traffic_src = "kernel changed since the counters were taken"
            else:
                traffic = t["families"][r["fam"]]["bytes_per_run"]
                traffic_src = "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated"
        cpu = cpu_baseline_lobpcg(c, 20) if (rank == 0 and not args.no_cpu_baseline) else None
        A = c["A"]
        fam = r["fam"]
        out = {
            "metric": METRIC_LOBPCG, "value": round(r["value"], 2), "unit": "LOBPCG iterations/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(1e3 * r["wall"] / args.steps, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
            "config": {"workload": f"LOBPCG: {c['k']} {c['which']} eigenpairs of the variable-coefficient Poisson "
                                   f"matrix 1024x1024 (kappa=exp(GRF) seed 0), tol {c['tol']}, X0[r]~N(0,1) "
                                   "seed 3+r, + Hellmann-Feynman gradient of sum(lambda)",
                       "n": A.n_rows, "nnz": A.nnz, "k": c["k"], "which": c["which"], "tol": c["tol"],
                       "parallelism": "none (1 GPU)", "method": "lobpcg"},
            "iterations": r["info"]["iterations"], "state": r["info"]["state_name"],
            "kernels": {kk: {"launches": v["launches"], "total_ms": round(v["total_ms"], 3),
                             "avg_us": round(1e3 * v["total_ms"] / v["launches"], 3) if v["launches"] else None,
                             "algorithmic_bytes": v["bytes"] or None}
                        for kk, v in r["tq"].items() if v["launches"]},
            "roofline": {"bound": "hbm", "kernel": f"{fam} ({', '.join(LOBPCG_FAMILIES[fam])}), all launches of one run",
                         "achieved": round(r["achieved"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(r["achieved"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
                         "traffic_source": traffic_src, "traffic_unit": "bytes per run (all launches)",
                         "bytes_per_launch": None, "bytes_per_run": r["tq"][fam]["bytes"],
                         "run_ms": round(r["tq"][fam]["total_ms"], 3)},
            "cpu_baseline": cpu,
        }
        if rank == 0:
            print(json.dumps(out), flush=True)
        return 0
    if args.workload == "poisson_list64":
        import workloads as W
        c = W.config(args.workload)
        r = run_list(args, c, S, torch, dev)
        if args.calibrate_copy:
            calibrate_copy(torch, dev)
        traffic, traffic_src = read_traffic(args.workload, "bytes_per_step")
        cpu = cpu_baseline_list(c, 150) if (rank == 0 and not args.no_cpu_baseline) else None
        n_tot = sum(A.n_rows for A in c["items"])
        out = {
            "metric": METRIC_LIST, "value": round(r["value"], 2), "unit": "CG iters/s (summed over items)",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(1e3 * r["wall"] / args.steps, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f64", "data": "synthetic",
            "config": {"workload": "SparseTensorList of 64 five-point Poisson grids, sides 64, 67, ..., 253 "
                                   "(distinct patterns), b_i~N(0,1) seed i, CG to 1e-8 + adjoint",
                       "items": len(c["items"]), "rows": n_tot, "rtol": c["rtol"], "parallelism": "none (1 GPU)",
                       "method": "list"},
            "iterations_per_step": {"forward_sum": sum(r["fi"]), "adjoint_sum": sum(r["bi"]),
                                    "forward_max": max(r["fi"]), "adjoint_max": max(r["bi"])},
            "kernels": {kk: {"launches": v["launches"],
                             "avg_us": round(1e3 * v["total_ms"] / v["launches"], 3) if v["launches"] else None}
                        for kk, v in r["tq"].items() if v["launches"]},
            "hbm_gbps_per_iteration": round(r["iter_gbps"], 1),
            "roofline": {"bound": "hbm", "kernel": "k_cg_spmv (list mode), all launches of one step",
                         "achieved": round(r["achieved"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(r["achieved"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
                         "traffic_source": traffic_src, "traffic_unit": "bytes per step (all launches)",
                         "bytes_per_launch": None,
                         "bytes_per_step": r["spmv_bytes"], "spmv_ms_per_step": round(r["spmv_ms"], 3)},
            "cpu_baseline": cpu,
        }
        if rank == 0:
            print(json.dumps(out), flush=True)
        return 0
    if args.ceiling_sweep:
        print(json.dumps({"ceiling_sweep": measure_ceiling(S, torch, dev, sweep=True)}), flush=True)
        return 0
    w = make_workload(args.workload, dev)
    method = w["method"]
    if method == "eigsh":
        r = run_eigsh(args, w, S, torch)
        if args.calibrate_copy:
            calibrate_copy(torch, dev)
        traffic, traffic_src = read_traffic(args.workload, "bytes_per_run")
        cpu = cpu_baseline_eigsh(w, 40) if (rank == 0 and not args.no_cpu_baseline) else None
        out = {
            "metric": METRIC_EIGSH, "value": round(r["value"], 2), "unit": "Lanczos steps/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(1e3 * r["wall"] / args.steps, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
            "data": "synthetic",
            "config": {"workload": w["desc"], "n": w["n"], "nnz": w["nnz"], "k": w["k"], "which": w["which"],
                       "tol": w["tol"], "max_dim": w["max_dim"], "max_iter": w["max_iter"],
                       "parallelism": "none (1 GPU)", "method": "eigsh"},
            "lanczos_steps": r["info"]["iterations"], "restarts": r["info"]["restarts"],
            "state": r["info"]["state_name"],
            "kernels": {kk: {"launches": v["launches"],
                             "avg_us": round(1e3 * v["total_ms"] / v["launches"], 3) if v["launches"] else None}
                        for kk, v in r["tq"].items() if v["launches"]},
            "bytes_model": r["bm"],
            "lz_spmv_gbps": round(r["spmv_gbps"], 1),
            "roofline": {"bound": "hbm",
                         "kernel": "Lanczos reorthogonalization (k_lz_three, k_lz_dots, k_lz_reduce, k_lz_axpy, "
                                   "k_lz_next), all launches of one run",
                         "achieved": round(r["achieved"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(r["achieved"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
                         "traffic_source": traffic_src, "traffic_unit": "bytes per run (all launches)",
                         "bytes_per_launch": None, "bytes_per_run": r["bm"]["lz_orth_total"],
                         "run_ms": round(r["orth_ms"], 3)},
            "cpu_baseline": cpu,
        }
        if rank == 0:
            print(json.dumps(out), flush=True)
        return 0
    r = measure_cg(args, w, S, torch, args.steps, args.warmup)
    if args.calibrate_copy:
        calibrate_copy(torch, dev)
    ceiling = measure_ceiling(S, torch, dev) if not args.no_ceiling else None
    if not args.no_ceiling and cache_resident(r["w"]) and not r["bicg"] and not r["an"]["split"]:
        rf0 = iteration_roofline(r)
        r["ceiling_resident"] = measure_ceiling_resident(S, torch, dev, rf0["bm"]["cg_spmv"],
                                                         rf0["bm"]["cg_update"])
    big = None
    if args.workload == "poisson1024" and not args.no_big and args.fixed_iters == 0 and not args.jacobi:
        # the metric's second configuration, 169M DOF (500 + 500 fixed iterations), timed
        # beside the 1M headline in the same run
        del w
        torch.cuda.empty_cache()
        wb = make_workload("poisson13000", dev)
        rb = measure_cg(args, wb, S, torch, args.big_steps, 1)
        big = cg_summary(rb, ceiling, args)
        del wb, rb
        torch.cuda.empty_cache()
    cpu = None
    if rank == 0 and not args.no_cpu_baseline:
        # a BiCGStab iteration is two products: half as many keep the sample's CPU time
        cpu = cpu_baseline(r["w"], max(1, args.cpu_iters // 2) if r["bicg"] else args.cpu_iters)
    out = cg_line(r, args, ceiling, cpu)
    if big is not None:
        out["poisson13000"] = big
    if rank == 0:
        print(json.dumps(out), flush=True)
    return 0


# ------------------------------------------------------------------------------ CG measurement
def measure_cg(args, w, S, torch, steps: int, warmup: int) -> dict:
    """Time `steps` solve + adjoint steps of workload w (after `warmup` untimed ones),
    then time every kernel of one more step with HIP events on the library's stream."""
    n, nnz, B = w["n"], w["nnz"], w["batch"]
    method = w["method"]
    bicg = method == "bicgstab"
    # csr_create (device validation and analysis of the pattern) is timed on its own,
    # outside the steps
    torch.cuda.synchronize()
    tc0 = time.perf_counter()
    h = S.csr_create(w["rp"], w["col"], symmetric=w["symmetric"])
    torch.cuda.synchronize()
    create_ms = 1e3 * (time.perf_counter() - tc0)
    an = S.csr_analysis(h)
    if bicg:
        spmv_kernel = "k_cg_spmv (BiCGStab modes: v = A p, t = A s)"
        schedule = "BiCGStab: p update, v = A p, s, t = A s, update (adjoint on the device transpose)"
    elif an["band_stride"] > 0 and an["diagonals"] > 0:
        spmv_kernel = "k_cg_spmv_dia"
        schedule = (f"fused, banded SpMV on the diagonal layout (line stride {an['band_stride']}, "
                    f"{an['diagonals']} diagonals)")
    elif an["band_stride"] > 0:
        spmv_kernel, schedule = "k_cg_spmv_band", f"fused, banded SpMV (line stride {an['band_stride']})"
    elif an["split"] and B >= 8 and B % 4 == 0 and nnz < 2 ** 31:
        spmv_kernel = "k_gcg_spmv"
        schedule = "split, grouped batch (4 systems interleaved per element; k_gcg_pupd, k_gcg_spmv)"
    elif an["split"]:
        spmv_kernel, schedule = "k_cg_spmv", "split (k_cg_pupd forms p_k, the SpMV gathers it)"
    else:
        spmv_kernel, schedule = "k_cg_spmv", "fused"
    # the plain and banded SpMV (CG and BiCGStab) read 16-bit column offsets where the
    # handle has them; the grouped kernels read the 32-bit columns unless their operand
    # window is on (below)
    col_bytes = 4 if spmv_kernel == "k_gcg_spmv" else an["col_bits"] // 8
    dia_nd = an["diagonals"] if spmv_kernel == "k_cg_spmv_dia" else 0
    rp_bytes = 4 if nnz < 2 ** 31 else 8      # the row pointers the kernels read
    rp_stated = w["rp"].element_size()        # the row-pointer width the workload hands in
    if args.fixed_iters > 0:
        w["max_iter"], w["fixed"], w["rtol"] = args.fixed_iters, True, 0.0
    opts = S.cg_opts(rtol=w["rtol"], max_iter=w["max_iter"], fixed=w["fixed"], jacobi=args.jacobi,
                     method=method)
    vals, b = w["vals"], w["b"]

    def step():
        x, info = S.solve(h, vals, b, opts)
        g = loss_grad(w, x)
        gb, gv, binfo = S.solve_backward(h, vals, x, g, opts)
        return x, gb, gv, info, binfo

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    infos, marks = [], []
    for _ in range(steps):
        _, _, _, info, binfo = step()
        infos.append((info, binfo))
        em = torch.cuda.Event(enable_timing=True)   # per-step marks on the stream, no sync
        em.record(stream)
        marks.append(em)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [e0.elapsed_time(marks[0])] + [marks[i - 1].elapsed_time(marks[i]) for i in range(1, len(marks))]
    fwd_it = [sum(s["iterations"] for s in S.read_info(i)) for i, _ in infos]
    bwd_it = [sum(s["iterations"] for s in S.read_info(bi)) for _, bi in infos]
    max_fwd = max(s["iterations"] for s in S.read_info(infos[-1][0]))
    max_bwd = max(s["iterations"] for s in S.read_info(infos[-1][1]))
    total_it = sum(fwd_it) + sum(bwd_it)

    # Kernel timing: the same solve + backward once more with per-launch HIP events on
    # the library's stream, fixed at the measured iteration counts so every timed
    # launch is a working one.
    S.timing.reset()
    S.timing.enable(True)
    fo = S.cg_opts(rtol=0.0, max_iter=max_fwd, fixed=True, jacobi=args.jacobi, method=method)
    bo = S.cg_opts(rtol=0.0, max_iter=max_bwd, fixed=True, jacobi=args.jacobi, method=method)
    x, _ = S.solve(h, vals, b, fo)
    S.solve_backward(h, vals, x, loss_grad(w, x), bo)
    S.timing.collect()
    S.timing.enable(False)
    tq = S.timing.query()
    torch.cuda.synchronize()
    if spmv_kernel == "k_gcg_spmv" and S.csr_analysis(h)["group_window"] > 0:
        # the windowed grouped SpMV (known after the first grouped solve) reads 16-bit
        # column offsets
        col_bytes = 2
        schedule += "; operand in an LDS window, 16-bit column offsets"
    del x, h
    return dict(w=w, an=an, bicg=bicg, spmv_kernel=spmv_kernel, schedule=schedule, col_bytes=col_bytes, dia_nd=dia_nd,
                rp_bytes=rp_bytes, rp_stated=rp_stated, steps=steps, warmup=warmup, wall=wall, create_ms=create_ms,
                step_ms=step_ms,
                event_ms=e0.elapsed_time(e1) / steps, fwd_it=fwd_it, bwd_it=bwd_it, total_it=total_it, tq=tq)


def iteration_roofline(r) -> dict:
    """Roofline of one CG iteration (every kernel of it: SpMV, update, and the p update
    of the split schedule), HIP-event timed.

    frac: the bytes of the iteration model with V = 9 vector passes, 4-byte column
    indices and the workload's stated row-pointer width (B 8 nnz + 4 nnz + rp (n + 1)
    + 72 n B), over the iteration's time, over 8 TB/s.  frac_bytes_moved: the bytes the
    kernels actually read and write (16-bit column offsets where the handle has them,
    the 32-bit row-pointer copy, the split schedule's extra pass), same time.
    frac_spmv_only: the SpMV's own bytes over its own time."""
    w, tq = r["w"], r["tq"]
    n, nnz, B = w["n"], w["nnz"], w["batch"]

    def avg_ms(key):
        return tq[key]["total_ms"] / max(tq[key]["launches"], 1)

    if r["bicg"]:
        bm = bytes_model_bicgstab(n, nnz, B, r["rp_bytes"], r["col_bytes"])
        spmv_ms, spmv_bytes = avg_ms("bs_spmv"), bm["bs_spmv"]
        iter_ms = 2 * spmv_ms + 3 * avg_ms("bs_vec")
        v9 = bm["iteration"]   # BiCGStab: its own model (two products, 14 vector passes)
    else:
        bm = bytes_model(n, nnz, B, r["rp_bytes"], split=r["an"]["split"], col_bytes=r["col_bytes"],
                         dia_nd=r["dia_nd"])
        spmv_ms, spmv_bytes = avg_ms("cg_spmv"), bm["cg_spmv"]
        iter_ms = spmv_ms + avg_ms("cg_update") + (avg_ms("cg_pupd") if r["an"]["split"] else 0.0)
        v9 = bytes_model_v9(n, nnz, B, r["rp_stated"])
    gbps = lambda by, ms: by / (ms * 1e-3) / 1e9
    achieved = gbps(v9, iter_ms)
    return dict(bm=bm, v9=v9, iter_ms=iter_ms, spmv_ms=spmv_ms, spmv_bytes=spmv_bytes, achieved=achieved,
                moved_gbps=gbps(bm["iteration"], iter_ms), spmv_gbps=gbps(spmv_bytes, spmv_ms))


def cache_resident(w) -> bool:
    """Whether one iteration's working set fits the 256 MB Infinity Cache."""
    return (12 * w["nnz"] + 52 * w["n"]) * w["batch"] < 200e6


def cg_summary(r, ceiling, args) -> dict:
    """The measured numbers of one CG workload (headline fields and its roofline)."""
    w = r["w"]
    B = w["batch"]
    rf = iteration_roofline(r)
    traffic, traffic_src = read_traffic(w["name"], "bytes_per_iteration")
    ms_step = 1e3 * r["wall"] / r["steps"]
    resident = cache_resident(w)
    roof = {"bound": "hbm",
            "kernel": ("one BiCGStab iteration (two products, three streaming kernels)" if r["bicg"] else
                       "one CG iteration: " + r["spmv_kernel"] + " + k_cg_update"
                       + (" + k_cg_pupd" if r["an"]["split"] else "")),
            "achieved": round(rf["achieved"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(rf["achieved"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "traffic_source": traffic_src, "traffic_unit": "HBM bytes per iteration (all kernels of it)",
            "bytes_model": ("BiCGStab: two products + 14 vector passes" if r["bicg"] else
                            "V=9: 8 nnz B + 4 nnz + rp (n+1) + 72 n B, 4-byte columns, "
                            f"rp = {r['rp_stated']} B as stated"),
            "bytes_per_iteration": rf["v9"], "iteration_us": round(1e3 * rf["iter_ms"], 3),
            "frac_bytes_moved": round(rf["moved_gbps"] / HBM_PEAK_GBPS, 4),
            "bytes_moved_per_iteration": rf["bm"]["iteration"],
            "frac_spmv_only": round(rf["spmv_gbps"] / HBM_PEAK_GBPS, 4),
            "spmv_us": round(1e3 * rf["spmv_ms"], 3), "spmv_bytes": rf["spmv_bytes"],
            "cache_resident": bool(resident)}
    if ceiling:
        roof["ceiling_gbps"] = {"spmv_mix": ceiling["spmv_mix"]["gbps"], "triad": ceiling["triad"]["gbps"]}
        # the iteration's bytes moved against the same-run streaming rate of its own mix:
        # the SpMV's bytes at the SpMV-mix ceiling plus the update's at the triad ceiling
        if not r["bicg"] and not r["an"]["split"]:
            t_ceil = (rf["bm"]["cg_spmv"] / ceiling["spmv_mix"]["gbps"] +
                      rf["bm"]["cg_update"] / ceiling["triad"]["gbps"]) / 1e9
            roof["frac_of_ceiling"] = round(t_ceil / (rf["iter_ms"] * 1e-3), 4)
    cr = r.get("ceiling_resident")
    if cr:
        # a cache-resident iteration against plain streams of its own sizes: the SpMV
        # mix moving the SpMV's bytes plus the triad moving the update's, each launch timed
        roof["resident_ceiling"] = cr
        roof["frac_of_resident_ceiling"] = round(
            (cr["spmv_mix"]["us"] + cr["triad"]["us"]) / (1e3 * rf["iter_ms"]), 4)
    return {"workload": w["desc"], "n": w["n"], "nnz": w["nnz"], "batch": B,
            "row_ptr": f"int{8 * r['rp_stated']} (kernels read int{8 * r['rp_bytes']})",
            "col_idx_read": ("none (diagonal layout)" if r["dia_nd"] else f"int{8 * r['col_bytes']}"),
            "rtol": w["rtol"], "fixed_iterations": w["fixed"],
            "cg_schedule": r["schedule"], "steps": r["steps"], "warmup": r["warmup"],
            "ms_per_step": round(ms_step, 4), "solve_adjoint_ms": round(ms_step, 4),
            "csr_create_ms": round(r["create_ms"], 3),
            "step_ms_median": (round(statistics.median(r["step_ms"]), 4) if r.get("step_ms") else None),
            "iterations_per_step": {"forward": r["fwd_it"][-1], "adjoint": r["bwd_it"][-1]},
            "iters_per_s": round(r["total_it"] / r["wall"], 2),
            "hbm_gbps_per_iteration": round(rf["achieved"], 1),
            "hbm_gbps_moved_per_iteration": round(rf["moved_gbps"], 1),
            "event_ms_per_step": round(r["event_ms"], 4),
            "kernels": {k: {"launches": v["launches"],
                            "avg_us": round(1e3 * v["total_ms"] / v["launches"], 3) if v["launches"] else None}
                        for k, v in r["tq"].items() if v["launches"]},
            "bytes_model": rf["bm"], "roofline": roof}


def cg_line(r, args, ceiling, cpu) -> dict:
    w = r["w"]
    sm = cg_summary(r, ceiling, args)
    out = {
        "metric": METRIC_BICGSTAB if r["bicg"] else METRIC,
        "value": sm["iters_per_s"],
        "unit": "BiCGStab iters/s" if r["bicg"] else "CG iters/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": r["warmup"],
        "ms_per_step": sm["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": w["desc"], "n": w["n"], "nnz": w["nnz"], "batch": w["batch"],
                   "row_ptr": sm["row_ptr"], "col_idx_read": sm["col_idx_read"], "rtol": w["rtol"],
                   "fixed_iterations": w["fixed"], "parallelism": "none (1 GPU)",
                   "cg_schedule": r["schedule"], "preconditioner": "jacobi" if args.jacobi else "none",
                   "method": w["method"]},
    }
    for k in ("iterations_per_step", "solve_adjoint_ms", "step_ms_median", "csr_create_ms", "hbm_gbps_per_iteration",
              "hbm_gbps_moved_per_iteration",
              "event_ms_per_step", "kernels", "bytes_model", "roofline"):
        out[k] = sm[k]
    if ceiling:
        out["ceiling"] = ceiling
    out["device"] = device_info()
    out["cpu_baseline"] = cpu
    return out


def device_info() -> dict:
    """The GPU the line was measured on (figures vary from box to box)."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1)}


# ------------------------------------------------------------------------------ ceiling
# Streaming probes (sla_probe_stream): (reads, writes) per element of each mix, and the
# variants (16-byte accesses in flight per thread and array, non-temporal hint,
# workgroups per CU) whose best rate is reported.
# Every variant is timed (about 0.2 s for all mixes): the reported rate of a mix is its
# best over all 24.
CEILING_MIXES = {"read": (1, 0), "write": (0, 1), "copy": (1, 1), "triad": (2, 1), "spmv_mix": (10, 3)}
CEILING_SWEEP = [(u, nt, bpc) for u in (1, 2, 4) for nt in (1, 0) for bpc in (1, 2, 4, 8)]


def _probe_best(lib, L, bufs, part, stream, torch, nr: int, nw: int, n: int, sweep: bool) -> dict:
    """Best rate of one read/write mix over n doubles per array, over the variants."""
    import ctypes as C
    ins = (C.c_void_p * max(nr, 1))(*[bufs[i].data_ptr() for i in range(nr)])
    outs = (C.c_void_p * max(nw, 1))(*[bufs[nr + i].data_ptr() for i in range(nw)])
    best = None
    for (u, nt, bpc) in (CEILING_SWEEP if sweep else CEILING_SWEEP[:1]):
        def launch():
            L.check(lib.sla_probe_stream(nr, nw, ins, outs, n, u, nt, bpc, part.data_ptr(), stream.cuda_stream))
        launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbps = 8.0 * n * (nr + nw) / (ms * 1e-3) / 1e9
        if best is None or gbps > best["gbps"]:
            best = {"gbps": round(gbps, 1), "unroll": u, "nontemporal": nt, "blocks_per_cu": bpc,
                    "us": round(1e3 * ms, 2), "bytes": 8 * n * (nr + nw)}
    return best


def measure_ceiling(S, torch, dev, sweep: bool = True, elems: int = 1 << 26) -> dict:
    """Bandwidth of plain coalesced streams on this GPU, in this run: for each mix the
    best rate (bytes read + written / event-timed launch) over the variants.  Arrays of
    `elems` doubles (512 MiB each by default: every mix streams far past the 256 MB
    Infinity Cache); the SpMV mix uses arrays a quarter as long (13 of them)."""
    from differentiable_sparse_linear_spmv_amd import _lib as L
    lib = L.load()
    bufs = [torch.empty(elems, dtype=torch.float64, device=dev) for _ in range(13)]
    for bb in bufs:
        bb.fill_(1.0)
    part = torch.zeros(8 * 1024, dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()
    out = {}
    for name, (nr, nw) in CEILING_MIXES.items():
        n = elems // 4 if nr + nw > 4 else elems
        out[name] = _probe_best(lib, L, bufs, part, stream, torch, nr, nw, n, sweep)
    del bufs, part
    torch.cuda.empty_cache()
    out["frac_of_peak"] = {k: round(v["gbps"] / HBM_PEAK_GBPS, 4) for k, v in out.items()}
    return out


def measure_ceiling_resident(S, torch, dev, spmv_bytes: int, update_bytes: int) -> dict:
    """The same probes at the sizes of one cache-resident CG iteration: the SpMV mix (10
    arrays read, 3 written) moving the SpMV's bytes, and the triad moving the update's.
    The arrays fit the Infinity Cache, as the iteration's working set does, so this is
    the rate plain streams of that size reach (launch and ramp included), not HBM's."""
    from differentiable_sparse_linear_spmv_amd import _lib as L
    lib = L.load()
    n_spmv = max(1024, int(spmv_bytes) // (8 * 13)) & ~1   # the probes take an even length
    n_upd = max(1024, int(update_bytes) // (8 * 3)) & ~1
    bufs = [torch.empty(max(n_spmv, n_upd), dtype=torch.float64, device=dev) for _ in range(13)]
    for bb in bufs:
        bb.fill_(1.0)
    part = torch.zeros(8 * 1024, dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()
    out = {"spmv_mix": _probe_best(lib, L, bufs, part, stream, torch, 10, 3, n_spmv, True),
           "triad": _probe_best(lib, L, bufs, part, stream, torch, 2, 1, n_upd, True)}
    del bufs, part
    torch.cuda.empty_cache()
    return out

if __name__ == "__main__":
    sys.exit(main())
