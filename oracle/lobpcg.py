"""LOBPCG eigensolver for symmetric sparse matrices -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this module; the HIP library never does and shares no code with it.

The pages name LOBPCG beside Lanczos as an eigensolver behind ``.eigsh`` (torch-sla,
paperpeel page, section 4.3, note to Table 5; the API of section 3.1) and print no
steps.  This is the method of Knyazev ("Toward the optimal preconditioned eigensolver:
locally optimal block preconditioned conjugate gradient method", SIAM J. Sci. Comput.
23(2), 2001), without a preconditioner, with the basis of every Rayleigh-Ritz step kept
orthonormal (Hetmaniuk and Lehoucq, "Basis selection in LOBPCG", J. Comput. Phys.
218, 2006), so that the small eigenproblem is a standard symmetric one:

    X = orth(X0^T)  (n x k);  AX = A X
    Rayleigh-Ritz on X:  H = X^T AX,  (theta, Y) = wanted k eigenpairs of H,
                         X = X Y,  AX = AX Y;   no P yet
    for it = 0, 1, ...:
        R = AX - X diag(theta);  res_r = |R_r|
        active r: res_r > tol |theta_r|;  none active -> CONVERGED after `it` iterations
        it == max_iter -> MAX_ITER
        W = R[:, active], made orthonormal against X:  twice W = W - X (X^T W),
            then orth(W)
        P = P[:, active] (if any), made orthonormal against [X, W] the same way
        a block whose orth() fails is left out of this iteration
        AW = A W; AP follows P through the same combinations
        S = [X, W, P] (orthonormal), AS = [AX, AW, AP]
        H = S^T AS, symmetrized (H + H^T) / 2; (theta, Y) = wanted k eigenpairs of H
        X = S Y, AX = AS Y
        P = S[:, k:] Y[k:, :],  AP = AS[:, k:] Y[k:, :]   (the part of the step
            outside the old X: Knyazev's conjugate direction)

orth(Z): every column scaled to unit norm (the residuals of different Ritz pairs
differ by orders of magnitude), then Cholesky QR twice (G = Z^T Z = R^T R, Z = Z R^-1);
it fails when a column is zero or a pivot of the Cholesky factorization is not above
1e-14 times the largest diagonal entry of G (numerically dependent columns).  AZ is
carried through the same scaling, R^-1 and projections (A is linear), so every SpMV is
applied to a W block only.

With jacobi=True the residuals are preconditioned before they enter the basis,
W = T R[:, active] with Knyazev's preconditioner T = D^-1 (D the stored diagonal of A,
applied as a product with the reciprocals 1 / a_ii); every a_ii must be stored,
finite and positive.

The eigenvalues returned are the Ritz values from the wanted end; the vectors are
unit Ritz vectors, signed so that <u_r, X0[r]> >= 0.  SpMV is the oracle's own
(sla_oracle.c); Gram products, Cholesky, triangular solves and the small symmetric
eigenproblem are library primitives (numpy / LAPACK).
"""
from __future__ import annotations

import numpy as np

from . import CONVERGED, MAX_ITER, _f64, spmv

ORTH_PIVOT = 1e-14


def _block_spmv(A, Z, vals):
    out = np.empty_like(Z)
    for c in range(Z.shape[1]):
        out[:, c] = spmv(A, np.ascontiguousarray(Z[:, c]), vals=vals)
    return out


def _orth(Z, AZ=None):
    """Columns scaled to unit norm, then Cholesky QR twice; returns (Z, AZ) with
    Z^T Z = I, or None when a column is zero or a pivot fails."""
    nrm = np.sqrt(np.sum(Z * Z, axis=0))
    if not np.all(nrm > 0.0):
        return None
    Z = Z / nrm
    if AZ is not None:
        AZ = AZ / nrm
    for _ in range(2):
        G = Z.T @ Z
        G = 0.5 * (G + G.T)
        m = G.shape[0]
        L = np.zeros_like(G)
        gmax = float(np.max(np.diag(G))) if m else 0.0
        for j in range(m):   # Cholesky G = L L^T with the pivot test
            d = G[j, j] - L[j, :j] @ L[j, :j]
            if not d > ORTH_PIVOT * gmax:
                return None
            L[j, j] = np.sqrt(d)
            for i in range(j + 1, m):
                L[i, j] = (G[i, j] - L[i, :j] @ L[j, :j]) / L[j, j]
        Rinv = np.linalg.inv(L.T)
        Z = Z @ Rinv
        if AZ is not None:
            AZ = AZ @ Rinv
    return Z, AZ


def _project(Z, AZ, B, AB):
    """Twice Z = Z - B (B^T Z) against the orthonormal block B (AZ alike)."""
    for _ in range(2):
        C = B.T @ Z
        Z = Z - B @ C
        if AZ is not None:
            AZ = AZ - AB @ C
    return Z, AZ


def _wanted(H, k, which):
    w, V = np.linalg.eigh(0.5 * (H + H.T))
    idx = np.arange(len(w) - 1, len(w) - 1 - k, -1) if which == "largest" else np.arange(k)
    return w[idx], V[:, idx]


def jacobi_reciprocals(A, vals=None) -> np.ndarray:
    """1 / a_ii for every row; ValueError unless each a_ii is stored, finite and > 0."""
    v = A.vals if vals is None else _f64(vals)
    rp = A.row_ptr.astype(np.int64)
    d = np.full(A.n_rows, np.nan)
    for i in range(A.n_rows):
        for e in range(rp[i], rp[i + 1]):
            if A.col[e] == i:
                d[i] = v[e]
    if not np.all(np.isfinite(d) & (d > 0.0)):
        raise ValueError("Jacobi needs every diagonal entry stored, finite and positive")
    return 1.0 / d


def lobpcg(A, k: int, X0, which: str = "largest", tol: float = 1e-8, max_iter: int = 1000, vals=None,
           jacobi: bool = False) -> dict:
    """Returns dict(evals [k], evecs [k, n], iterations, state, res [k] (true residual
    norms |A u - theta u| of the returned pairs, from the last check), blocks (per
    iteration: the widths of W and P used))."""
    if which not in ("largest", "smallest"):
        raise ValueError(which)
    n = A.n_rows
    X0 = np.atleast_2d(_f64(X0))
    if X0.shape != (k, n) or not 1 <= k or 3 * k > n:
        raise ValueError("need X0 of shape [k, n] with 3 k <= n")
    tinv = jacobi_reciprocals(A, vals) if jacobi else None
    q = _orth(X0.T.copy())
    if q is None:
        raise ValueError("start block is rank deficient")
    X = q[0]
    AX = _block_spmv(A, X, vals)
    theta, Y = _wanted(X.T @ AX, k, which)
    X, AX = X @ Y, AX @ Y
    P = AP = None
    it = 0
    blocks = []
    while True:
        R = AX - X * theta
        res = np.sqrt(np.sum(R * R, axis=0))
        active = res > tol * np.abs(theta)
        if not active.any() or it == max_iter:
            state = CONVERGED if not active.any() else MAX_ITER
            break
        it += 1
        W = R[:, active] * tinv[:, None] if jacobi else R[:, active]
        W, _ = _project(W, None, X, AX)
        ow = _orth(W)
        W = ow[0] if ow is not None else None
        AW = _block_spmv(A, W, vals) if W is not None else None
        basis, abasis = [X], [AX]
        if W is not None:
            basis.append(W)
            abasis.append(AW)
        Pn = APn = None
        if P is not None:
            Bq, ABq = np.hstack(basis), np.hstack(abasis)
            Pp, APp = _project(P[:, active], AP[:, active], Bq, ABq)
            op = _orth(Pp, APp)
            if op is not None:
                Pn, APn = op
                basis.append(Pn)
                abasis.append(APn)
        blocks.append((0 if W is None else W.shape[1], 0 if Pn is None else Pn.shape[1]))
        S, AS = np.hstack(basis), np.hstack(abasis)
        theta, Y = _wanted(S.T @ AS, k, which)
        X, AX = S @ Y, AS @ Y
        P, AP = S[:, k:] @ Y[k:, :], AS[:, k:] @ Y[k:, :]
    U = X.T.copy()
    for r in range(k):
        U[r] /= np.sqrt(U[r] @ U[r])
        if U[r] @ X0[r] < 0.0:
            U[r] = -U[r]
    return dict(evals=theta.copy(), evecs=U, iterations=it, state=state, res=res, blocks=blocks)
