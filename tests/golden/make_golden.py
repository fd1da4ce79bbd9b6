"""Write the full-size expected values used by the GPU parity tests.

Every value here comes from the CPU oracle (oracle/) on the seeded workloads
(workloads/): nothing is taken from the HIP library.  For each benchmark workload
it records the oracle's iteration counts, residual and right-hand-side norms, and
the solution, adjoint and matrix gradient at seeded sample positions (the full
vectors are too large to store as fixtures).

    python tests/golden/make_golden.py [name ...]      # default: all

poisson64       CG to 1e-10 + adjoint of 0.5|x|^2 (whole vectors stored).
poisson1024     CG to 1e-8 + adjoint of 0.5|x|^2.
varcoef2048     CG to 1e-8 + adjoint of sum (x - x_target)^2.
fem256x256      256 systems to 1e-8 + adjoint of sum_b 0.5|x_b|^2 (iteration counts of
                every system; samples of 8 systems).
poisson13000    the first 20 fixed iterations forward and adjoint (the full 500 are
                beyond a CPU fixture): residual history and samples of x, lambda, grads.
convdiff1024    BiCGStab to 1e-8 on the nonsymmetric convection-diffusion matrix and on
                its transpose in the adjoint of 0.5|x|^2, with the true residuals.
Runs take from seconds (poisson64) to tens of minutes (varcoef2048, fem256x256).
"""
from __future__ import annotations

import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

NSAMP = 256


def samples(n: int, seed: int) -> np.ndarray:
    return np.sort(np.random.default_rng(seed).choice(n, size=min(NSAMP, n), replace=False))


def loss_grad(c, x, s=0):
    if c["loss"] == "sq_target":
        return 2.0 * (x - c["x_target"])
    return x.copy()


def one_system(A, b, vals, c, want_full=False, g_of=None):
    opts = dict(rtol=c["rtol"], atol=c["atol"], max_iter=c["max_iter"], fixed=c["fixed"],
                method=c.get("method", "cg"))
    f = O.cg(A, b, vals=vals, **opts)
    g = loss_grad(c, f["x"]) if g_of is None else g_of(f["x"])
    bw = O.solve_backward(A, f["x"], g, symmetric=c.get("symmetric", True), vals=vals, **opts)
    out = dict(iterations=f["iterations"], state=f["state"], res_norm=f["res_norm"],
               rhs_norm=f["rhs_norm"], x_norm=float(np.linalg.norm(f["x"])),
               adj_iterations=bw["iterations"], adj_state=bw["state"], adj_res_norm=bw["res_norm"],
               adj_rhs_norm=bw["rhs_norm"], lam_norm=float(np.linalg.norm(bw["lam"])),
               gvals_norm=float(np.linalg.norm(bw["gvals"])))
    ix, ik = samples(A.n_rows, 11), samples(A.nnz, 12)
    out.update(ix=ix.tolist(), ik=ik.tolist(), x=f["x"][ix].tolist(), lam=bw["lam"][ix].tolist(),
               gvals=bw["gvals"][ik].tolist())
    if c.get("method") == "bicgstab":
        # true residuals of the oracle's solutions (the stop test is on the recurrence)
        out.update(true_res=float(np.linalg.norm(b - O.spmv(A, f["x"], vals=vals))),
                   adj_true_res=float(np.linalg.norm(g - O.spmv_transposed(A, bw["lam"], vals=vals))))
    if want_full:
        out.update(x_full=f["x"].tolist(), lam_full=bw["lam"].tolist())
    return out


_FEM = None   # per worker process: the batch is generated once


def _fem_system(args):
    global _FEM
    s, rtol = args
    if _FEM is None:
        _FEM = W.config("fem256x256")
    c = _FEM
    A, b = c["A"], c["b"]
    r = one_system(A, b[s], A.vals[s], c)
    return s, r


def make(name: str) -> dict:
    t0 = time.time()
    if name == "fem256x256":
        c = W.config(name)
        B = c["A"].batch
        keep = set(np.random.default_rng(13).choice(B, 8, replace=False).tolist())
        with ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            res = dict(ex.map(_fem_system, [(s, c["rtol"]) for s in range(B)]))
        out = dict(name=name, batch=B, iterations=[res[s]["iterations"] for s in range(B)],
                   adj_iterations=[res[s]["adj_iterations"] for s in range(B)],
                   states=[res[s]["state"] for s in range(B)],
                   systems={str(s): res[s] for s in sorted(keep)})
    elif name == "poisson13000":
        N, K = 13000, 20
        A = W.poisson5(N, index64=True)
        b = W.rhs_normal(N * N, 0)
        f = O.cg(A, b, rtol=0.0, max_iter=K, fixed=True, history=True)
        bw = O.solve_backward(A, f["x"], f["x"], symmetric=True, rtol=0.0, max_iter=K, fixed=True)
        ix, ik = samples(A.n_rows, 11), samples(A.nnz, 12)
        out = dict(name=name, fixed_iterations=K, history=f["history"].tolist(),
                   x_norm=float(np.linalg.norm(f["x"])), lam_norm=float(np.linalg.norm(bw["lam"])),
                   ix=ix.tolist(), ik=ik.tolist(), x=f["x"][ix].tolist(), lam=bw["lam"][ix].tolist(),
                   gvals=bw["gvals"][ik].tolist(), adj_res_norm=bw["res_norm"])
    else:
        c = W.config(name)
        A = c["A"]
        out = dict(name=name, **one_system(A, c["b"], A.vals, c, want_full=(name == "poisson64")))
    out["oracle_seconds"] = round(time.time() - t0, 1)
    out["source"] = ("tests/golden/make_golden.py: CPU oracle (oracle/) on the seeded workloads "
                     "of workloads/; sample positions from numpy default_rng(11) for rows and "
                     "default_rng(12) for stored entries")
    return out


def main(names):
    for name in names:
        out = make(name)
        p = os.path.join(HERE, f"{name}.json")
        with open(p, "w") as f:
            json.dump(out, f)
        print(f"{name}: wrote {p} in {out['oracle_seconds']} s", flush=True)


if __name__ == "__main__":
    ALL = ["poisson64", "poisson1024", "fem256x256", "poisson13000", "varcoef2048", "convdiff1024"]
    main(sys.argv[1:] or ALL)
