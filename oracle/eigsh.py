"""Lanczos eigensolver (eigsh) for symmetric sparse matrices and the Hellmann-Feynman
eigenvalue gradient -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this module; the HIP library never does and shares no code with it.

What it computes, from torch-sla (Differentiable Sparse Linear Algebra with Adjoint
Solvers and Sparse Tensor Parallelism for PyTorch):
  * ``eigsh``   the k extreme eigenpairs of a symmetric A by Lanczos, one of the two
                eigensolvers behind the pages' .eigsh entry point (paperpeel page,
                section 4.3, note to Table 5; the API of section 3.1).
  * ``eigsh_grad``  dL/dA_ij = sum_m dL/dlambda_m v_m[i] v_m[j] on the stored entries:
                the Hellmann-Feynman gradient of a unit eigenvector's eigenvalue
                (gist.science Japanese summary, Methodology item 2, eigenvalue bullet;
                paperpeel section 4.3: an O(nnz) outer product, no linear solve).

The Lanczos steps (the pages name the method but print no steps; this is the textbook
form with full reorthogonalization):
    v_0 = v0 / |v0|;  beta_{-1} = 0
    for j = 0, 1, ...:
        w = A v_j;  alpha_j = <v_j, w>
        w = w - alpha_j v_j - beta_{j-1} v_{j-1}
        twice: w = w - V_j (V_j^T w)          (full reorthogonalization against
                                                v_0 .. v_j, "twice is enough")
        beta_j = |w|
        T_j = tridiag(beta_0..beta_{j-1}; alpha_0..alpha_j; beta_0..beta_{j-1})
        once j + 1 >= k: Ritz pairs (theta_i, s_i) of T_j; the k wanted ones (largest
        or smallest algebraic) have residuals |A u_i - theta_i u_i| = beta_j |s_i[j]|;
        stop when every one is <= tol |theta_i|, or beta_j = 0 (the Krylov space is
        invariant: the Ritz pairs are exact), or j + 1 = max_dim (MAX_ITER); beta_j
        counts as 0 when it is at most sqrt(n) eps |T_j| (|T_j| the largest row sum of
        |T_j| with beta_j), the rounding level of a reorthogonalized w
        v_{j+1} = w / beta_j
    u_i = V_j s_i, normalized, signed so that <u_i, v0> >= 0.
The eigenvalues returned are the Ritz values theta_i, sorted from the wanted end.
A Krylov space that becomes invariant before it holds k Ritz values is BREAKDOWN.
The eigen-decomposition of the small tridiagonal T_j is a library primitive
(scipy.linalg.eigh_tridiagonal, LAPACK); SpMV and inner products are the oracle's own
(sla_oracle.c).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import eigh_tridiagonal

from . import BREAKDOWN, CONVERGED, MAX_ITER, _f64, dot, pattern_outer, spmv


def eigsh(A, k: int, v0, which: str = "largest", tol: float = 1e-10, max_dim: int | None = None,
          vals=None) -> dict:
    """Returns dict(evals [k], evecs [k, n], iterations (Krylov dimension), state,
    res_est [k] (beta_j |s_i[j]|), alpha, beta)."""
    if which not in ("largest", "smallest"):
        raise ValueError(which)
    n = A.n_rows
    m_max = min(n, max_dim or n)
    if not 1 <= k <= m_max:
        raise ValueError("need 1 <= k <= max_dim <= n")
    v = _f64(v0)
    V = np.zeros((m_max + 1, n))
    V[0] = v / np.sqrt(dot(v, v))
    alpha, beta = [], []
    for j in range(m_max):
        w = spmv(A, V[j], vals=vals)
        a = dot(V[j], w)
        w = w - a * V[j]
        if j > 0:
            w = w - beta[j - 1] * V[j - 1]
        for _ in range(2):
            h = V[: j + 1] @ w
            w = w - V[: j + 1].T @ h
        b = float(np.sqrt(dot(w, w)))
        alpha.append(a)
        beta.append(b)
        m = j + 1
        # |T| by its largest Gershgorin row sum (beta_j included): beta_j at the rounding
        # level of the reorthogonalized w means the Krylov space is (numerically) invariant
        tnorm = max(abs(alpha[l]) + abs(beta[l]) + (abs(beta[l - 1]) if l > 0 else 0.0) for l in range(m))
        if b <= np.sqrt(n) * np.finfo(np.float64).eps * tnorm:
            b = 0.0
            beta[-1] = 0.0
        if m >= k or b == 0.0:
            theta, S = eigh_tridiagonal(np.array(alpha), np.array(beta[:-1]))
            if m < k:                     # invariant before k Ritz values exist
                return dict(evals=np.full(k, np.nan), evecs=np.zeros((k, n)), iterations=m,
                            state=BREAKDOWN, res_est=np.full(k, np.nan), alpha=np.array(alpha),
                            beta=np.array(beta))
            idx = np.arange(m - 1, m - 1 - k, -1) if which == "largest" else np.arange(k)
            res = b * np.abs(S[m - 1, idx])
            done = bool(np.all(res <= tol * np.abs(theta[idx])))
            if done or b == 0.0 or m == m_max:
                U = S[:, idx].T @ V[:m]
                for i in range(k):
                    U[i] /= np.sqrt(dot(U[i], U[i]))
                    if dot(U[i], v) < 0.0:
                        U[i] = -U[i]
                state = CONVERGED if (done or b == 0.0) else MAX_ITER
                return dict(evals=theta[idx].copy(), evecs=U, iterations=m, state=state, res_est=res,
                            alpha=np.array(alpha), beta=np.array(beta))
        V[j + 1] = w / b
    raise AssertionError("unreachable")


def eigsh_grad(A, evecs, g_evals) -> np.ndarray:
    """dL/dvals[e] = sum_m g_m u_m[row(e)] u_m[col(e)] over the wanted eigenpairs, for
    every stored entry (no symmetrisation, as for the linear adjoint)."""
    out = np.zeros(A.nnz)
    for m in range(evecs.shape[0]):
        out = out + float(g_evals[m]) * pattern_outer(A, evecs[m], evecs[m], sign=1.0)
    return out
