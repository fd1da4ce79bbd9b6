"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.

This module builds matrices and right-hand sides only.  It holds none of the
solver's arithmetic (no SpMV, no CG, no adjoint): both the CPU oracle and the
HIP path consume what it returns, and neither side imports the other.

Workloads are stand-ins for the 2-D Poisson benchmarks of the torch-sla paper
(paperpeel page, section 4.1 "Single-GPU scalability" and section 4.2
"Adjoint vs. Naive Backpropagation"), and for the batched shared-pattern
SparseTensor described in section 3.1 ("Typed sparse-tensor hierarchy").

Readings where the pages are silent (stencil scale, ordering, coefficient
field, mesh, loss) are stated in each generator's docstring.
All randomness is ``numpy.random.default_rng(seed)`` (PCG64).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "CSR", "poisson5", "poisson5_torch", "varcoef_poisson5", "gaussian_random_field",
    "fem_p1_batched", "convdiff5", "graph_laplacian", "rhs_uniform", "rhs_normal", "config",
]


@dataclasses.dataclass
class CSR:
    """Compressed sparse rows.  ``vals`` is ``[nnz]`` or ``[B, nnz]`` (shared pattern)."""
    n_rows: int
    n_cols: int
    row_ptr: np.ndarray   # int32 or int64, [n_rows + 1]
    col: np.ndarray       # int32, [nnz]
    vals: np.ndarray      # float64, [nnz] or [B, nnz]

    @property
    def nnz(self) -> int:
        return int(self.col.shape[0])

    @property
    def batch(self) -> int:
        return 1 if self.vals.ndim == 1 else int(self.vals.shape[0])


def _poisson5_pattern_np(N: int):
    """Row pointer and columns of the 5-point stencil on an N x N interior grid.

    Unknown (a, c) (grid row a, grid column c) is number a*N + c.  Within a row the
    columns ascend: a*N+c-N, -1, 0, +1, +N, with neighbours outside the grid
    dropped (homogeneous Dirichlet boundary eliminated).
    """
    n = N * N
    idx = np.arange(n, dtype=np.int64)
    a, c = idx // N, idx % N
    valid = [a > 0, c > 0, np.ones(n, bool), c < N - 1, a < N - 1]
    offs = [-N, -1, 0, 1, N]
    cnt = np.zeros(n, np.int64)
    for m in valid:
        cnt += m
    row_ptr = np.zeros(n + 1, np.int64)
    np.cumsum(cnt, out=row_ptr[1:])
    nnz = int(row_ptr[-1])
    col = np.empty(nnz, np.int32)
    slot = np.zeros(n, np.int64)
    pos_of = []
    for m, o in zip(valid, offs):
        rows = idx[m]
        pos = row_ptr[rows] + slot[rows]
        col[pos] = (rows + o).astype(np.int32)
        slot[rows] += 1
        pos_of.append((m, pos))
    return row_ptr, col, pos_of


def poisson5(N: int, index64: bool = False) -> CSR:
    """Constant-coefficient 5-point Poisson matrix, unscaled (diagonal 4, neighbours -1).

    The pages fix a five-point stencil with homogeneous Dirichlet data on a 2-D
    grid but give no scale; the integer form keeps every product exact for
    integer vectors and leaves iteration counts and relative errors unchanged.
    """
    row_ptr, col, pos_of = _poisson5_pattern_np(N)
    vals = np.empty(col.shape[0], np.float64)
    for k, (_, pos) in enumerate(pos_of):
        vals[pos] = 4.0 if k == 2 else -1.0
    if not index64:
        row_ptr = row_ptr.astype(np.int32)
    return CSR(N * N, N * N, row_ptr, col, vals)


def poisson5_torch(N: int, device, index64: bool = True):
    """Same matrix as :func:`poisson5`, built with torch ops directly on ``device``.

    Used for the 13000 x 13000 grid, whose 845M stored entries are cheaper to
    build in device memory than to copy over.  Returns (row_ptr, col, vals).
    """
    import torch
    n = N * N
    idx = torch.arange(n, dtype=torch.int64, device=device)
    a = torch.div(idx, N, rounding_mode="floor")
    c = idx - a * N
    valid = [a > 0, c > 0, None, c < N - 1, a < N - 1]
    del a, c
    cnt = torch.ones(n, dtype=torch.int64, device=device)
    for m in valid:
        if m is not None:
            cnt += m
    row_ptr = torch.zeros(n + 1, dtype=torch.int64, device=device)
    torch.cumsum(cnt, 0, out=row_ptr[1:])
    del cnt
    nnz = int(row_ptr[-1].item())
    col = torch.empty(nnz, dtype=torch.int32, device=device)
    vals = torch.empty(nnz, dtype=torch.float64, device=device)
    slot = torch.zeros(n, dtype=torch.int64, device=device)
    for m, o, v in zip(valid, (-N, -1, 0, 1, N), (-1.0, -1.0, 4.0, -1.0, -1.0)):
        rows = idx if m is None else idx[m]
        pos = row_ptr[rows] + slot[rows]
        col[pos] = (rows + o).to(torch.int32)
        vals[pos] = v
        slot[rows] += 1
        del rows, pos
    del slot, idx, valid
    if not index64:
        row_ptr = row_ptr.to(torch.int32)
    return row_ptr, col, vals


def gaussian_random_field(M: int, h: float, ell: float, sigma: float, rng) -> np.ndarray:
    """Stationary Gaussian field on an M x M node grid with spacing h.

    Covariance sigma^2 * exp(-r^2 / (2 ell^2)).  Sampled by circulant embedding
    on a periodic grid twice as large (so the torus never wraps a correlation
    length onto the sampled square): white noise is filtered in Fourier space
    by the square root of the embedded covariance's spectrum, which gives the
    exact marginal variance sigma^2 wherever that spectrum is non-negative.
    """
    P = 2 * M
    d = np.minimum(np.arange(P), P - np.arange(P)) * h
    cov = sigma * sigma * np.exp(-(d[:, None] ** 2 + d[None, :] ** 2) / (2.0 * ell * ell))
    lam = np.fft.fft2(cov).real
    lam = np.maximum(lam, 0.0)
    w = rng.standard_normal((P, P))
    g = np.fft.ifft2(np.sqrt(lam) * np.fft.fft2(w)).real
    return g[:M, :M].copy()


def varcoef_poisson5(N: int, seed: int = 0, ell: float = 0.1, sigma: float = 1.0,
                     kappa: np.ndarray | None = None):
    """Variable-coefficient -div(kappa grad u) = f, 5-point finite differences.

    kappa = exp(g) with g a Gaussian random field (squared-exponential kernel)
    sampled on the (N+2)^2 grid of nodes including the boundary, h = 1/(N+1).
    Face coefficients are harmonic means 2 kP kQ / (kP + kQ) for every pair of
    adjacent nodes (boundary pairs included).  Row P: diagonal = sum of its four
    face coefficients, off-diagonal -k_PQ for interior neighbours Q; Dirichlet
    u = 0 is eliminated.  The system is scaled by h^2, so b = h^2 f with
    f ~ U[0, 1].  kappa == 1 gives exactly the matrix of :func:`poisson5`.

    Returns (CSR, b, rng) -- rng continues the seed-``seed`` stream.
    """
    rng = np.random.default_rng(seed)
    h = 1.0 / (N + 1)
    if kappa is None:
        g = gaussian_random_field(N + 2, h, ell, sigma, rng)
        kappa = np.exp(g)
    assert kappa.shape == (N + 2, N + 2)
    K = kappa

    def hm(p, q):
        return 2.0 * p * q / (p + q)

    inner = K[1:-1, 1:-1]
    kN = hm(inner, K[:-2, 1:-1])   # face to grid row a-1
    kS = hm(inner, K[2:, 1:-1])    # face to grid row a+1
    kW = hm(inner, K[1:-1, :-2])   # face to column c-1
    kE = hm(inner, K[1:-1, 2:])    # face to column c+1
    diag = (kN + kS) + (kW + kE)
    row_ptr, col, pos_of = _poisson5_pattern_np(N)
    vals = np.empty(col.shape[0], np.float64)
    n = N * N
    idx = np.arange(n)
    for slot, (m, pos) in enumerate(pos_of):
        rows = idx[m]
        src = (kN, kW, diag, kE, kS)[slot].reshape(-1)[rows]
        vals[pos] = src if slot == 2 else -src
    f = rng.uniform(0.0, 1.0, n)
    b = (h * h) * f
    return CSR(n, n, row_ptr.astype(np.int32), col, vals), b, rng


def _tri_mesh(nv: int, rng, jitter: float):
    """Jittered structured triangulation of the unit square with nv x nv vertices.

    Vertex (i, j) sits at (j h, i h), h = 1/(nv-1); interior vertices move by
    U[-jitter h, jitter h] in each coordinate.  Every cell is split along its
    (i, j)-(i+1, j+1) diagonal.  Returns coordinates [nv*nv, 2] and triangles
    [2 (nv-1)^2, 3] in natural vertex numbering.
    """
    h = 1.0 / (nv - 1)
    ii, jj = np.meshgrid(np.arange(nv), np.arange(nv), indexing="ij")
    xy = np.stack([jj * h, ii * h], axis=-1).reshape(-1, 2).astype(np.float64)
    d = rng.uniform(-jitter * h, jitter * h, size=(nv, nv, 2))
    interior = np.zeros((nv, nv), bool)
    interior[1:-1, 1:-1] = True
    d[~interior] = 0.0
    xy = xy + d.reshape(-1, 2)
    v = np.arange(nv * nv).reshape(nv, nv)
    v00, v01 = v[:-1, :-1].ravel(), v[:-1, 1:].ravel()
    v10, v11 = v[1:, :-1].ravel(), v[1:, 1:].ravel()
    t1 = np.stack([v00, v01, v11], axis=1)
    t2 = np.stack([v00, v11, v10], axis=1)
    tris = np.concatenate([t1, t2], axis=0)
    return xy, tris


def fem_p1_batched(nv: int = 256, B: int = 256, seed: int = 0, jitter: float = 0.3,
                   mass: float = 1e-3, kappa_range=(0.5, 2.0)):
    """Batch of P1 finite-element systems K(kappa_b) + mass * M sharing one pattern.

    One jittered triangulated nv x nv-vertex mesh; vertex ids are a seeded
    random permutation of the natural order (unstructured gathers).  Every
    vertex is a degree of freedom (natural boundary), and the mass term makes
    each system SPD.  Element stiffness kappa_e |T| grad(phi_i).grad(phi_j) with
    kappa_e ~ U[kappa_range] per element and per system; consistent mass
    |T|/12 (1 + delta_ij).  |T| is the unsigned area.  Draw order from the one
    seeded stream: jitter, permutation, kappa [B, n_elem], b [B, n].

    Returns (CSR with vals [B, nnz], b [B, n]).
    """
    rng = np.random.default_rng(seed)
    xy, tris = _tri_mesh(nv, rng, jitter)
    n = nv * nv
    perm = rng.permutation(n)          # natural id -> stored id
    tris = perm[tris]
    xy_p = np.empty_like(xy)
    xy_p[perm] = xy
    ne = tris.shape[0]
    kap = rng.uniform(kappa_range[0], kappa_range[1], size=(B, ne))
    b = rng.standard_normal((B, n))

    P = xy_p[tris]                     # [ne, 3, 2]
    e1 = P[:, 1] - P[:, 0]
    e2 = P[:, 2] - P[:, 0]
    det = e1[:, 0] * e2[:, 1] - e1[:, 1] * e2[:, 0]
    area = 0.5 * np.abs(det)
    # gradients of the barycentric basis functions: grad phi_i = R(edge opposite i) / det
    opp = np.stack([P[:, 2] - P[:, 1], P[:, 0] - P[:, 2], P[:, 1] - P[:, 0]], axis=1)
    grad = np.stack([opp[..., 1], -opp[..., 0]], axis=-1) / det[:, None, None]
    Ke = area[:, None, None] * np.einsum("eid,ejd->eij", grad, grad)   # [ne, 3, 3]
    Me = (area / 12.0)[:, None, None] * (np.ones((3, 3)) + np.eye(3))[None]

    # pattern: vertex-adjacency from the triangles, canonical CSR (sorted columns)
    rows = np.repeat(tris, 3, axis=1).reshape(-1)
    cols = np.tile(tris, (1, 3)).reshape(-1)
    key = rows.astype(np.int64) * n + cols
    ukey, inv = np.unique(key, return_inverse=True)
    urow = (ukey // n).astype(np.int64)
    ucol = (ukey % n).astype(np.int32)
    nnz = ukey.shape[0]
    row_ptr = np.zeros(n + 1, np.int64)
    np.cumsum(np.bincount(urow, minlength=n), out=row_ptr[1:])
    vals = np.empty((B, nnz), np.float64)
    Ke_f = Ke.reshape(-1)
    Me_f = Me.reshape(-1)
    mass_part = np.bincount(inv, weights=Me_f, minlength=nnz)
    for s in range(B):
        stiff = np.bincount(inv, weights=(kap[s][:, None] * Ke.reshape(ne, 9)).reshape(-1),
                            minlength=nnz)
        vals[s] = stiff + mass * mass_part
    del Ke_f
    csr = CSR(n, n, row_ptr.astype(np.int32), ucol, vals)
    return csr, b


def convdiff5(N: int, wind=100.0, shift: float = 0.0, index64: bool = False) -> CSR:
    """Nonsymmetric 2-D convection-diffusion matrix: -Lap u + w . grad u on the unit
    square, N x N interior grid (h = 1 / (N + 1)), homogeneous Dirichlet data, the
    5-point Laplacian plus first-order upwind convection, scaled by h^2 like
    :func:`poisson5` (kappa = 1 gives exactly that matrix when w = 0).

    The pages support nonsymmetric systems through BiCGStab but name no nonsymmetric
    workload; this is the textbook stand-in.  The wind is the recirculating flow
    w = W (2 Y (1 - X^2), -2 X (1 - Y^2)) with X = 2 x - 1, Y = 2 y - 1, evaluated at
    each unknown.  Upwinding gives, at unknown P with neighbours S, W, E, N,
        A_PP = 4 + h (|w_x| + |w_y|),  A_PW = -1 - h max(w_x, 0),
        A_PE = -1 - h max(-w_x, 0),     A_PS = -1 - h max(w_y, 0),
        A_PN = -1 - h max(-w_y, 0),
    an M-matrix (nonsingular, weakly diagonally dominant) whose nonsymmetric part
    grows with W.  Same pattern and ordering as :func:`poisson5`.  ``wind``: W, or a
    sequence of W values for a shared-pattern batch (vals [B, nnz]).  ``shift`` adds a
    reaction term c u (c = shift, on the h^2-scaled diagonal): c >= 1 makes the matrix
    strictly diagonally dominant and well conditioned (a few tens of iterations).
    """
    row_ptr, col, pos_of = _poisson5_pattern_np(N)
    n = N * N
    h = 1.0 / (N + 1)
    idx = np.arange(n, dtype=np.int64)
    a, c = idx // N, idx % N
    X = 2.0 * (c + 1) * h - 1.0           # column index c runs along x
    Y = 2.0 * (a + 1) * h - 1.0           # grid row a runs along y
    winds = np.atleast_1d(np.asarray(wind, dtype=np.float64))
    vals = np.empty((winds.shape[0], col.shape[0]), np.float64)
    for bi, W in enumerate(winds):
        wx = W * 2.0 * Y * (1.0 - X * X)
        wy = -W * 2.0 * X * (1.0 - Y * Y)
        # neighbour order of the pattern: S (i - N), W (i - 1), P, E (i + 1), N (i + N)
        coef = [-1.0 - h * np.maximum(wy, 0.0), -1.0 - h * np.maximum(wx, 0.0),
                (4.0 + shift) + h * (np.abs(wx) + np.abs(wy)),
                -1.0 - h * np.maximum(-wx, 0.0), -1.0 - h * np.maximum(-wy, 0.0)]
        for k, (m, pos) in enumerate(pos_of):
            vals[bi, pos] = coef[k][m]
    if np.ndim(wind) == 0:
        vals = vals[0]
    if not index64:
        row_ptr = row_ptr.astype(np.int32)
    return CSR(n, n, row_ptr, col, vals)


def rhs_uniform(n: int, seed: int = 0, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    return np.random.default_rng(seed).uniform(lo, hi, n)


def rhs_normal(n: int, seed: int = 0) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal(n)


def graph_laplacian(n: int, avg_deg: float = 8.0, gamma: float = 2.5, seed: int = 0) -> CSR:
    """Weighted graph Laplacian + identity of a random power-law graph: an SPD system
    with a skewed row-length distribution (a few rows with thousands of entries, most
    with a handful).  The pages name graph Laplacians as the next validation target
    (paperpeel page, section 5 "Limitations and future work"); this is the stand-in.

    Graph (Chung-Lu): node i has weight w_i = (i + 1)^(-1 / (gamma - 1)); n avg_deg / 2
    edges draw both endpoints independently with probability proportional to w; self
    loops and repeated pairs are dropped, so degrees follow a power law with exponent
    gamma.  Each edge gets a weight c_e ~ U[0.5, 1.5].  The node ids are a random
    permutation (the hubs are scattered over the rows).  Matrix: A_ij = -c_e for every
    edge e = {i, j}, A_ii = 1 + sum of the weights at i, so A = L + I (L the weighted
    Laplacian, positive semidefinite) and every row of A sums to 1.  One seeded stream
    draws the endpoints, the weights and the permutation, in that order.  Columns ascend
    within a row; int32 indices.
    """
    rng = np.random.default_rng(seed)
    w = (np.arange(n, dtype=np.float64) + 1.0) ** (-1.0 / (gamma - 1.0))
    p = w / w.sum()
    m = int(n * avg_deg / 2)
    u = rng.choice(n, size=m, p=p)
    v = rng.choice(n, size=m, p=p)
    keep = u != v
    lo, hi = np.minimum(u[keep], v[keep]), np.maximum(u[keep], v[keep])
    key = np.unique(lo.astype(np.int64) * n + hi)
    lo, hi = key // n, key % n
    c = rng.uniform(0.5, 1.5, key.shape[0])
    perm = rng.permutation(n)
    lo, hi = perm[lo], perm[hi]
    rows = np.concatenate([lo, hi, np.arange(n)])
    cols = np.concatenate([hi, lo, np.arange(n)])
    deg = np.bincount(lo, weights=c, minlength=n) + np.bincount(hi, weights=c, minlength=n)
    vals = np.concatenate([-c, -c, 1.0 + deg])
    order = np.lexsort((cols, rows))
    rows, cols, vals = rows[order], cols[order], vals[order]
    rp = np.zeros(n + 1, np.int64)
    np.cumsum(np.bincount(rows, minlength=n), out=rp[1:])
    return CSR(n, n, rp.astype(np.int32), cols.astype(np.int32), vals)


# --------------------------------------------------------------------------------------
# The five benchmark workloads, by name.  Each returns a dict with the CSR, the
# right-hand side(s), the loss gradient rule and the solver settings.
# --------------------------------------------------------------------------------------
def config(name: str, scale: int | None = None) -> dict:
    """Named workloads.  ``scale`` overrides the grid size for reduced parity cases.

    poisson64      5-point Poisson, 64 x 64 interior grid, b ~ U[-1, 1] (seed 0),
                   rtol 1e-10, loss 0.5 |x|^2.
    poisson1024    same stencil, 1024 x 1024, b ~ N(0, 1) (seed 0), rtol 1e-8,
                   loss 0.5 |x|^2.
    varcoef2048    variable-coefficient Poisson on 2048 x 2048, kappa = exp(GRF),
                   f ~ U[0, 1] (seed 0), rtol 1e-8, loss sum (x - x_target)^2 with
                   x_target ~ U[0, 1] from seed 1.
    fem256x256     256 systems, P1 FEM Laplacian + 1e-3 mass on a jittered
                   256 x 256-vertex mesh, rtol 1e-8, loss sum_b 0.5 |x_b|^2.
    poisson13000   5-point Poisson on 13000 x 13000 (169M unknowns), int64 row
                   pointer, b ~ N(0, 1) (seed 0); 500 fixed CG iterations forward
                   and 500 in the adjoint, loss 0.5 |x|^2.
    eigsh_varcoef1024  the 8 largest eigenpairs of the varcoef matrix on 1024 x 1024
                   (kappa = exp(GRF), seed 0) by Lanczos to tol 1e-10 from v0 ~ N(0, 1)
                   (seed 3), and the Hellmann-Feynman gradient of sum(lambda).
    eigsh_tr_varcoef1024  the same with thick restart: a basis of 32 vectors (keep 20)
                   restarted until convergence.
    lobpcg_varcoef1024  the 8 largest eigenpairs of the same matrix by LOBPCG to tol
                   1e-8 from the start block X0[r] ~ N(0, 1) (seed 3 + r).
    poisson_list64 a SparseTensorList of 64 five-point Poisson grids of sides 64, 67, ...,
                   253 (distinct patterns, 1.7M rows in all), b_i ~ N(0, 1) seed i, CG to
                   1e-8 + adjoint of sum_i 0.5 |x_i|^2.
    graph1m        graph Laplacian + I of a power-law graph (:func:`graph_laplacian`,
                   2^20 nodes, average degree 8, exponent 2.5, seed 0): skewed row
                   lengths; b ~ N(0, 1) (seed 0), CG to 1e-8 + adjoint of 0.5 |x|^2.
    convdiff1024   nonsymmetric convection-diffusion (:func:`convdiff5`, W = 100) on
                   1024 x 1024, b ~ N(0, 1) (seed 0), BiCGStab to rtol 1e-8 forward and
                   on A^T in the adjoint, loss 0.5 |x|^2.
    """
    if name == "poisson64":
        N = scale or 64
        A = poisson5(N)
        return dict(name=name, A=A, b=rhs_uniform(N * N, 0), rtol=1e-10, atol=0.0,
                    max_iter=100000, fixed=False, loss="half_sq")
    if name == "poisson1024":
        N = scale or 1024
        A = poisson5(N)
        return dict(name=name, A=A, b=rhs_normal(N * N, 0), rtol=1e-8, atol=0.0,
                    max_iter=100000, fixed=False, loss="half_sq")
    if name == "varcoef2048":
        N = scale or 2048
        A, b, _ = varcoef_poisson5(N, seed=0)
        xt = np.random.default_rng(1).uniform(0.0, 1.0, N * N)
        return dict(name=name, A=A, b=b, x_target=xt, rtol=1e-8, atol=0.0,
                    max_iter=400000, fixed=False, loss="sq_target")
    if name == "fem256x256":
        nv, B = (scale or 256), 256
        if scale is not None:
            B = max(2, min(256, scale // 8))
        A, b = fem_p1_batched(nv=nv, B=B, seed=0)
        return dict(name=name, A=A, b=b, rtol=1e-8, atol=0.0, max_iter=100000,
                    fixed=False, loss="half_sq")
    if name == "convdiff1024":
        N = scale or 1024
        A = convdiff5(N, wind=100.0)
        return dict(name=name, A=A, b=rhs_normal(N * N, 0), rtol=1e-8, atol=0.0,
                    max_iter=100000, fixed=False, loss="half_sq", method="bicgstab",
                    symmetric=False)
    if name == "poisson_list64":
        sizes = [64 + 3 * i for i in range(64)]
        items = [poisson5(N) for N in sizes]
        return dict(name=name, items=items, b=[rhs_normal(A.n_rows, i) for i, A in enumerate(items)],
                    sizes=sizes, rtol=1e-8, atol=0.0, max_iter=100000, fixed=False, loss="half_sq",
                    method="list")
    if name in ("eigsh_varcoef1024", "eigsh_tr_varcoef1024"):
        N = scale or 1024
        A, _, _ = varcoef_poisson5(N, seed=0)
        c = dict(name=name, A=A, v0=rhs_normal(N * N, 3), k=8, which="largest", tol=1e-10,
                 method="eigsh", max_dim=0, max_iter=0, keep=0)
        if name == "eigsh_tr_varcoef1024":
            c.update(max_dim=32, max_iter=100000)
        return c
    if name == "lobpcg_varcoef1024":
        N = scale or 1024
        A, _, _ = varcoef_poisson5(N, seed=0)
        X0 = np.stack([rhs_normal(N * N, 3 + r) for r in range(8)])
        return dict(name=name, A=A, X0=X0, k=8, which="largest", tol=1e-8, max_iter=5000, method="lobpcg")
    if name == "graph1m":
        n = scale or (1 << 20)
        A = graph_laplacian(n, avg_deg=8.0, gamma=2.5, seed=0)
        return dict(name=name, A=A, b=rhs_normal(n, 0), rtol=1e-8, atol=0.0, max_iter=100000,
                    fixed=False, loss="half_sq")
    if name == "poisson13000":
        N = scale or 13000
        return dict(name=name, N=N, A=None, b=None, rtol=0.0, atol=0.0, max_iter=500,
                    fixed=True, loss="half_sq")
    raise KeyError(name)


def grid_of(n: int) -> int:
    N = int(math.isqrt(n))
    assert N * N == n
    return N
