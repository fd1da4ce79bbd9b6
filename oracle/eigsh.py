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
        the projected matrix with beta_j), the rounding level of a reorthogonalized w
        v_{j+1} = w / beta_j
    u_i = V_j s_i, normalized, signed so that <u_i, v0> >= 0.
The eigenvalues returned are the Ritz values theta_i, sorted from the wanted end.

Thick restart (Wu and Simon, "Thick-restart Lanczos method for large symmetric
eigenvalue problems", SIAM J. Matrix Anal. Appl. 22(2), 2000), when the step budget
max_iter exceeds the basis size max_dim: the stop test then runs when the basis is
full (and at an invariant space or the budget); if it fails, the basis restarts from
the `keep` Ritz vectors at the wanted end, u_i = V s_i, followed by the next Lanczos
vector v_m = w / beta.  The projected matrix of the new basis is diag(theta_i)
bordered by the couplings beta s_i[m-1] (the Lanczos relation restricted to the kept
vectors), and the first step after a restart removes those couplings instead of the
three-term pair.  Its small eigenproblem is then dense (numpy.linalg.eigh).
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
          vals=None, max_iter: int | None = None, keep: int | None = None) -> dict:
    """Returns dict(evals [k], evecs [k, n], iterations (Lanczos steps), state,
    res_est [k] (beta_j |s_i[j]|), restarts).

    max_iter > max_dim turns on thick restart: when the basis holds max_dim vectors
    the wanted-end `keep` Ritz vectors (default (max_dim + k) // 2) and the next
    Lanczos vector start a new basis, and the steps go on up to max_iter in all."""
    if which not in ("largest", "smallest"):
        raise ValueError(which)
    n = A.n_rows
    m_max = min(n, max_dim or n)
    total = max(m_max, max_iter or m_max)
    if not 1 <= k <= m_max:
        raise ValueError("need 1 <= k <= max_dim <= n")
    restart = total > m_max
    l_keep = keep or min(m_max - 1, max(k + 1, (m_max + k) // 2))
    if restart and not k <= l_keep < m_max:
        raise ValueError("need k <= keep < max_dim")
    eps = np.finfo(np.float64).eps
    v = _f64(v0)
    V = np.zeros((m_max + 1, n))
    V[0] = v / np.sqrt(dot(v, v))
    H = np.zeros((m_max + 1, m_max + 1))   # projected matrix of the current basis
    j0 = 0                                 # vectors kept at the last restart
    j = 0
    steps = 0
    restarts = 0
    while True:
        w = spmv(A, V[j], vals=vals)
        a = dot(V[j], w)
        w = w - a * V[j]
        if j > j0:
            w = w - H[j - 1, j] * V[j - 1]
        elif j0 > 0:                       # first step after a restart: the kept vectors
            for i in range(j0):
                w = w - H[i, j0] * V[i]
        for _ in range(2):
            h = V[: j + 1] @ w
            w = w - V[: j + 1].T @ h
        b = float(np.sqrt(dot(w, w)))
        steps += 1
        m = j + 1
        H[j, j] = a
        H[j, j + 1] = H[j + 1, j] = b
        # |T| by the largest row sum of the projected matrix, beta_j included
        tnorm = np.abs(H[:m, : m + 1]).sum(axis=1).max()
        if b <= np.sqrt(n) * eps * tnorm:
            b = 0.0
            H[j, j + 1] = H[j + 1, j] = 0.0
        check = (m >= k or b == 0.0) if not restart else (m == m_max or b == 0.0 or steps == total)
        if check:
            theta, S = np.linalg.eigh(H[:m, :m]) if restart else eigh_tridiagonal(np.diag(H)[:m],
                                                                                   np.diag(H, 1)[: m - 1])
            if m < k:                     # invariant before k Ritz values exist
                return dict(evals=np.full(k, np.nan), evecs=np.zeros((k, n)), iterations=steps,
                            state=BREAKDOWN, res_est=np.full(k, np.nan), restarts=restarts)
            order = np.arange(m - 1, -1, -1) if which == "largest" else np.arange(m)
            idx = order[:k]
            res = b * np.abs(S[m - 1, idx])
            done = bool(np.all(res <= tol * np.abs(theta[idx])))
            if done or b == 0.0 or steps == total or (not restart and m == m_max):
                U = S[:, idx].T @ V[:m]
                for i in range(k):
                    U[i] /= np.sqrt(dot(U[i], U[i]))
                    if dot(U[i], v) < 0.0:
                        U[i] = -U[i]
                state = CONVERGED if (done or b == 0.0) else MAX_ITER
                return dict(evals=theta[idx].copy(), evecs=U, iterations=steps, state=state, res_est=res,
                            restarts=restarts)
            if restart and m == m_max:
                # thick restart: the kept Ritz vectors, then the next Lanczos vector; the
                # projected matrix becomes diag(theta) bordered by the couplings beta s[m-1]
                kept = order[:l_keep]
                Ukeep = S[:, kept].T @ V[:m]
                nxt = w / b
                V[:] = 0.0
                V[:l_keep] = Ukeep
                V[l_keep] = nxt
                H[:] = 0.0
                for i, c in enumerate(kept):
                    H[i, i] = theta[c]
                    H[i, l_keep] = H[l_keep, i] = b * S[m - 1, c]
                j0 = j = l_keep
                restarts += 1
                continue
        V[j + 1] = w / b
        j += 1


def eigsh_grad(A, evecs, g_evals) -> np.ndarray:
    """dL/dvals[e] = sum_m g_m u_m[row(e)] u_m[col(e)] over the wanted eigenpairs, for
    every stored entry (no symmetrisation, as for the linear adjoint)."""
    out = np.zeros(A.nnz)
    for m in range(evecs.shape[0]):
        out = out + float(g_evals[m]) * pattern_outer(A, evecs[m], evecs[m], sign=1.0)
    return out
