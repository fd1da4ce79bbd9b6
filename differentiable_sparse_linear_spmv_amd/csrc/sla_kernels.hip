// sla_kernels.hip -- CDNA4 (gfx950) kernels of the sparse CG solve and its adjoint.
//
// What is computed follows torch-sla (Differentiable Sparse Linear Algebra with
// Adjoint Solvers and Sparse Tensor Parallelism for PyTorch): conjugate gradients
// driven by a CSR SpMV with the inner products <p,Ap> and <r,r> per iteration
// (paperpeel page, section 3.3 "Distributed Krylov solvers"), and the linear
// adjoint's matrix gradient -lambda_i x_j evaluated on the stored entries only
// (gist.science summaries, Methodology item 2, linear-systems bullet; paperpeel
// section 3.2.3 "Complexity": an O(nnz) outer product).
//
// How it is computed is this library's own design for MI355X:
//   * Two fused kernels per CG iteration.  k_cg_spmv forms p_k = r_k + beta p_{k-1}
//     on the fly for every gathered column (no separate p pass), applies the
//     deferred x update x_k = x_{k-1} + alpha_{k-1} p_{k-1} to its own rows, computes
//     q = A p_k and a partial p^T q.  k_cg_update forms alpha, r -= alpha q and a
//     partial r^T r.  Nine vector passes per iteration instead of eleven.
//   * Grid reductions are single-pass and deterministic: each workgroup writes one
//     partial; every workgroup of the next kernel sums the partials in the same
//     fixed order, so all of them hold bit-identical scalars.  Stop decisions and
//     the scalars alpha, beta stay in device memory; no host round trip per step.
//   * The SpMV stages each 256-row tile's values and columns through LDS with
//     coalesced loads, then one lane sums one row sequentially in ascending entry
//     order (the oracle's order, so row sums are bit-identical to it).  Tiles whose
//     entries exceed the LDS cap take a wave-per-row path with a fixed-order
//     shuffle reduction.
//   * Workgroups are remapped so that each of the 8 XCDs streams a contiguous band
//     of tiles: grid-neighbour rows (i +- N) are then read by the same XCD and
//     usually hit its L2 rather than another die's.
// All arithmetic is built with -ffp-contract=off: every product is rounded before
// it is added, as in the oracle, so elementwise updates match it exactly and only
// the order of the dot-product sums differs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sla_internal.h"

namespace sla {
namespace {

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = v + __shfl_xor(v, off, 64);
    return v;
}

// Sum over the workgroup; every thread gets the same value.  s_red: kBlock/64 doubles.
__device__ __forceinline__ double block_sum(double v, double* s_red)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s_red[w] = v;
    __syncthreads();
    const double t = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    __syncthreads();
    return t;
}

// Deterministic sum of G partials written by the previous kernel.
__device__ __forceinline__ double reduce_partials(const double* part, int G, double* s_red)
{
    double v = 0.0;
    for (int i = threadIdx.x; i < G; i += kBlock) v = v + part[i];
    return block_sum(v, s_red);
}

// Workgroup -> logical block.  Workgroups are dispatched round-robin over the 8
// XCDs; with G a multiple of 8, XCD x gets logical blocks [x G/8, (x+1) G/8), so
// at every grid-stride step it streams one contiguous band of tiles.
__device__ __forceinline__ int logical_block(int G, int remap)
{
    const int bx = blockIdx.x;
    if (remap && (G & 7) == 0) return (bx & 7) * (G >> 3) + (bx >> 3);
    return bx;
}

template <typename RP>
__device__ __forceinline__ int64_t ld_rp(const RP* rp, int64_t i)
{
    return static_cast<int64_t>(rp[i]);
}

// Gathered operand of the CG SpMV: p_k[c] = r_k[c] + beta * p_{k-1}[c]; p_0 = b.
struct GatherCG {
    const double* __restrict__ rin;
    const double* __restrict__ pprev;
    double beta;
    bool first;
    __device__ __forceinline__ double operator()(int64_t c) const
    {
        const double rv = rin[c];
        if (first) return rv;
        const double t = beta * pprev[c];
        return rv + t;
    }
};

struct GatherX {
    const double* __restrict__ x;
    __device__ __forceinline__ double operator()(int64_t c) const { return x[c]; }
};

// Row sums of one tile [row0, row0 + nr) for lane tid (0 for tid >= nr).  Contains
// the workgroup barriers of the LDS staging; every thread of the workgroup must call it.
template <typename RP, int CAP, typename G>
__device__ __forceinline__ double tile_rowsum(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                              const double* __restrict__ vals, int64_t row0, int nr,
                                              const G& g, double* s_val, int32_t* s_col)
{
    const int tid = threadIdx.x;
    const int64_t k0 = ld_rp(rp, row0);
    const int64_t k1 = ld_rp(rp, row0 + nr);
    const int64_t cnt = k1 - k0;
    double s = 0.0;
    if (cnt <= CAP) {
        constexpr int U = CAP / kBlock;
        double v[U];
        int32_t c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = tid + u * kBlock;
            if (j < cnt) {
                v[u] = vals[k0 + j];
                c[u] = col[k0 + j];
            }
        }
        int rs = 0, re = 0;
        if (tid < nr) {
            rs = static_cast<int>(ld_rp(rp, row0 + tid) - k0);
            re = static_cast<int>(ld_rp(rp, row0 + tid + 1) - k0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = tid + u * kBlock;
            if (j < cnt) {
                s_val[j] = v[u];
                s_col[j] = c[u];
            }
        }
        __syncthreads();
        for (int j0 = rs; j0 < re; j0 += 8) {
            double av[8], pv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                if (j < re) {
                    av[u] = s_val[j];
                    pv[u] = g(s_col[j]);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u < re) {
                    const double t = av[u] * pv[u];
                    s = s + t;
                }
            }
        }
        __syncthreads();
    } else {
        // Wave per row: lanes stride over the row's entries, fixed-order shuffle sum.
        const int lane = tid & 63;
        const int w = tid >> 6;
        double* s_q = s_val;   // nr <= kTile doubles, CAP >= kTile
        for (int rr = w; rr < nr; rr += kBlock / 64) {
            const int64_t a = ld_rp(rp, row0 + rr);
            const int64_t e = ld_rp(rp, row0 + rr + 1);
            double acc = 0.0;
            for (int64_t kk = a + lane; kk < e; kk += 64) {
                const double t = vals[kk] * g(col[kk]);
                acc = acc + t;
            }
            acc = wave_sum(acc);
            if (lane == 0) s_q[rr] = acc;
        }
        __syncthreads();
        if (tid < nr) s = s_q[tid];
        __syncthreads();
    }
    return s;
}

// ----------------------------------------------------------------------------------
// CG kernels.  Grid: (G, batch) workgroups of kBlock threads; logical block lb of
// system `sys` owns tiles lb, lb + G, lb + 2G, ...
// ----------------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_cg_init(CgArgs a)
{
    __shared__ double s_red[kBlock / 64];
    const int sys = blockIdx.y;
    const int lb = logical_block(a.G, a.xcd_remap);
    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const double* __restrict__ b = a.b + off;
    double* __restrict__ x = a.x + off;
    double rr = 0.0;
    for (int64_t t = lb; t < a.ntiles; t += a.G) {
        const int64_t i = t * kTile + threadIdx.x;
        if (i < a.n) {
            const double bv = b[i];
            x[i] = 0.0;
            const double u = bv * bv;
            rr = rr + u;
        }
    }
    rr = block_sum(rr, s_red);
    if (threadIdx.x == 0) {
        a.part_rho[static_cast<int64_t>(sys) * a.G + lb] = rr;
        if (lb == 0) a.st[sys].stop_iter = INT64_MAX;
        if (lb == 0 && sys == 0) *a.n_active = a.batch;
    }
}

template <typename RP, int CAP>
__global__ __launch_bounds__(kBlock) void k_cg_spmv(CgArgs a, int64_t k)
{
    __shared__ double s_val[CAP];
    __shared__ int32_t s_col[CAP];
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const int sys = blockIdx.y;
    SysState* st = a.st + sys;
    const int tid = threadIdx.x;
    // One read per workgroup, so the exit decision is uniform even while this
    // kernel's leading workgroup may be writing stop_iter = k.
    if (tid == 0) s_stop = st->stop_iter;
    __syncthreads();
    if (s_stop < k) return;   // stopped in an earlier kernel
    const int lb = logical_block(a.G, a.xcd_remap);
    const bool lead = (lb == 0 && tid == 0);
    const bool first = (k == 0);

    const double rho_k = reduce_partials(a.part_rho + static_cast<int64_t>(sys) * a.G, a.G, s_red);
    const double res = sqrt(rho_k);
    double thr, rhs;
    if (first) {
        rhs = res;
        thr = a.rtol * rhs;
        if (a.atol > thr) thr = a.atol;
    } else {
        thr = st->thr;
        rhs = st->rhs;
    }
    if (lead && a.hist) a.hist[static_cast<int64_t>(sys) * (a.max_iter + 1) + k] = res;

    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const double* __restrict__ pprev = ((k & 1) ? a.p0 : a.p1) + off;   // p_{k-1}
    double* __restrict__ pcur = ((k & 1) ? a.p1 : a.p0) + off;          // p_k
    double* __restrict__ x = a.x + off;
    const double alpha_prev = first ? 0.0 : st->alpha[(k - 1) & 1];

    int code = -1;
    if (!a.fixed && res <= thr) code = SLA_CONVERGED;
    else if (k >= a.max_iter) code = SLA_MAX_ITER;
    if (code >= 0) {
        // Stop: apply the deferred update x_k = x_{k-1} + alpha_{k-1} p_{k-1}.
        if (!first) {
            for (int64_t t = lb; t < a.ntiles; t += a.G) {
                const int64_t i = t * kTile + tid;
                if (i < a.n) {
                    const double tx = alpha_prev * pprev[i];
                    x[i] = x[i] + tx;
                }
            }
        }
        if (lead) {
            st->stop_iter = k;
            if (first) { st->rhs = rhs; st->thr = thr; }
            sla_cg_info inf;
            inf.iterations = k;
            inf.res_norm = res;
            inf.rhs_norm = rhs;
            inf.state = code;
            inf.reserved = 0;
            a.info[sys] = inf;
            atomicSub(a.n_active, 1);
        }
        return;
    }
    const double beta = first ? 0.0 : rho_k / st->rho[(k - 1) & 1];
    if (lead) {
        st->rho[k & 1] = rho_k;
        if (first) { st->thr = thr; st->rhs = rhs; }
    }

    const RP* __restrict__ rp = static_cast<const RP*>(a.row_ptr);
    const double* __restrict__ vals = a.vals + static_cast<int64_t>(sys) * a.nnz;
    const double* __restrict__ rin = (first ? a.b : a.r) + off;
    double* __restrict__ q = a.q + off;
    GatherCG g{rin, pprev, beta, first};
    double sig = 0.0;
    for (int64_t t = lb; t < a.ntiles; t += a.G) {
        const int64_t row0 = t * kTile;
        const int nr = static_cast<int>(min(static_cast<int64_t>(kTile), a.n - row0));
        const double s = tile_rowsum<RP, CAP>(rp, a.col, vals, row0, nr, g, s_val, s_col);
        if (tid < nr) {
            const int64_t i = row0 + tid;
            const double pi = g(i);
            pcur[i] = pi;
            q[i] = s;
            if (!first) {
                const double tx = alpha_prev * pprev[i];
                x[i] = x[i] + tx;
            }
            const double u = pi * s;
            sig = sig + u;
        }
    }
    sig = block_sum(sig, s_red);
    if (tid == 0) a.part_sigma[static_cast<int64_t>(sys) * a.G + lb] = sig;
}

__global__ __launch_bounds__(kBlock) void k_cg_update(CgArgs a, int64_t k)
{
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const int sys = blockIdx.y;
    SysState* st = a.st + sys;
    const int tid = threadIdx.x;
    if (tid == 0) s_stop = st->stop_iter;
    __syncthreads();
    if (s_stop <= k) return;
    const int lb = logical_block(a.G, a.xcd_remap);
    const bool lead = (lb == 0 && tid == 0);
    const double sigma = reduce_partials(a.part_sigma + static_cast<int64_t>(sys) * a.G, a.G, s_red);
    const double rho_k = st->rho[k & 1];
    if (!(sigma > 0.0)) {
        if (lead) {
            st->stop_iter = k;
            sla_cg_info inf;
            inf.iterations = k;
            inf.res_norm = sqrt(rho_k);
            inf.rhs_norm = st->rhs;
            inf.state = (sigma != sigma) ? SLA_NAN : SLA_NOT_SPD;
            inf.reserved = 0;
            a.info[sys] = inf;
            atomicSub(a.n_active, 1);
        }
        return;
    }
    const double alpha = rho_k / sigma;
    if (lead) st->alpha[k & 1] = alpha;
    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const double* __restrict__ rin = (k == 0 ? a.b : a.r) + off;
    const double* __restrict__ q = a.q + off;
    double* __restrict__ r = a.r + off;
    double rr = 0.0;
    for (int64_t t = lb; t < a.ntiles; t += a.G) {
        const int64_t i = t * kTile + tid;
        if (i < a.n) {
            const double tq = alpha * q[i];
            const double rn = rin[i] - tq;
            r[i] = rn;
            const double u = rn * rn;
            rr = rr + u;
        }
    }
    rr = block_sum(rr, s_red);
    if (tid == 0) a.part_rho[static_cast<int64_t>(sys) * a.G + lb] = rr;
}

// ----------------------------------------------------------------------------------
// y = A x (one tile per workgroup; grid (ntiles, batch))
// ----------------------------------------------------------------------------------
template <typename RP, int CAP>
__global__ __launch_bounds__(kBlock) void k_matvec(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                                   const double* __restrict__ vals, const double* __restrict__ x,
                                                   double* __restrict__ y, int64_t n_rows, int64_t nnz,
                                                   int64_t n_cols)
{
    __shared__ double s_val[CAP];
    __shared__ int32_t s_col[CAP];
    const int sys = blockIdx.y;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kTile;
    const int nr = static_cast<int>(min(static_cast<int64_t>(kTile), n_rows - row0));
    GatherX g{x + static_cast<int64_t>(sys) * n_cols};
    const double s = tile_rowsum<RP, CAP>(rp, col, vals + static_cast<int64_t>(sys) * nnz, row0, nr, g,
                                          s_val, s_col);
    if (static_cast<int>(threadIdx.x) < nr) y[static_cast<int64_t>(sys) * n_rows + row0 + threadIdx.x] = s;
}

// g[k] = sign * u[row(k)] * v[col(k)] over the stored entries of one tile; the row
// of entry k is found by binary search in the tile's row pointers (held in LDS), so
// entries are read and written coalesced whatever the row lengths.
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_pattern_outer(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                                          double sign, const double* __restrict__ u, int64_t us,
                                                          const double* __restrict__ v, int64_t vs,
                                                          double* __restrict__ g, int64_t n_rows, int64_t nnz)
{
    __shared__ int64_t s_rp[kTile + 1];
    __shared__ double s_u[kTile];
    const int sys = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kTile;
    const int nr = static_cast<int>(min(static_cast<int64_t>(kTile), n_rows - row0));
    for (int j = tid; j <= nr; j += kBlock) s_rp[j] = ld_rp(rp, row0 + j);
    if (tid < nr) s_u[tid] = u[static_cast<int64_t>(sys) * us + row0 + tid];
    __syncthreads();
    const int64_t k0 = s_rp[0], k1 = s_rp[nr];
    const double* __restrict__ vb = v + static_cast<int64_t>(sys) * vs;
    double* __restrict__ gb = g + static_cast<int64_t>(sys) * nnz;
    for (int64_t kk = k0 + tid; kk < k1; kk += kBlock) {
        int lo = 0, hi = nr;   // s_rp[lo] <= kk < s_rp[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_rp[mid] <= kk) lo = mid;
            else hi = mid;
        }
        const double t = s_u[lo] * vb[col[kk]];
        gb[kk] = sign * t;
    }
}

__global__ __launch_bounds__(kBlock) void k_gather_vals(const int64_t* __restrict__ perm,
                                                        const double* __restrict__ vals,
                                                        double* __restrict__ out, int64_t nnz)
{
    const int64_t base = static_cast<int64_t>(blockIdx.y) * nnz;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t kk = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; kk < nnz; kk += stride)
        out[base + kk] = vals[base + perm[kk]];
}

// ----------------------------------------------------------------------------------
// CSR validation and tile analysis
// ----------------------------------------------------------------------------------
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_validate(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                                     int64_t n_rows, int64_t n_cols, int64_t nnz,
                                                     int32_t* err, int32_t* tile_max)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (i == 0) {
        if (ld_rp(rp, 0) != 0 || ld_rp(rp, n_rows) != nnz) atomicOr(err, 1);
    }
    if (i < n_rows) {
        const int64_t a = ld_rp(rp, i), e = ld_rp(rp, i + 1);
        if (a > e || a < 0 || e > nnz) {
            atomicOr(err, 2);
        } else {
            int64_t prev = -1;
            for (int64_t kk = a; kk < e; ++kk) {
                const int64_t c = col[kk];
                if (c < 0 || c >= n_cols) atomicOr(err, 4);
                if (c <= prev) atomicOr(err, 8);
                prev = c;
            }
        }
        if ((i % kTile) == 0) {
            const int64_t last = min(i + kTile, n_rows);
            int64_t cnt = ld_rp(rp, last) - a;
            if (cnt > 0x7fffffff) cnt = 0x7fffffff;
            if (cnt > 0) atomicMax(tile_max, static_cast<int32_t>(cnt));
        }
    }
}

// ----------------------------------------------------------------------------------
// Transpose of the pattern: column histogram, exclusive scan, atomic scatter, then a
// per-row sort by original position (so A^T comes out canonical and deterministic).
// ----------------------------------------------------------------------------------
constexpr int kScanChunk = 2048;   // elements per workgroup in the scan (8 per thread)

__global__ __launch_bounds__(kBlock) void k_fill_i64(int64_t* p, int64_t n, int64_t v)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) p[i] = v;
}

__global__ __launch_bounds__(kBlock) void k_count_cols(const int32_t* __restrict__ col, int64_t nnz,
                                                       unsigned long long* cnt)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t kk = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; kk < nnz; kk += stride)
        atomicAdd(cnt + col[kk], 1ull);
}

// Exclusive scan of each kScanChunk chunk in place; chunk totals to sums (nullable).
__global__ __launch_bounds__(kBlock) void k_scan_chunks(int64_t* data, int64_t n, int64_t* sums)
{
    __shared__ int64_t s_t[kBlock];
    const int tid = threadIdx.x;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanChunk + tid * 8;
    int64_t v[8];
    int64_t tot = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        v[u] = (base + u < n) ? data[base + u] : 0;
        tot += v[u];
    }
    s_t[tid] = tot;
    __syncthreads();
    for (int off = 1; off < kBlock; off <<= 1) {   // Hillis-Steele inclusive scan of thread totals
        const int64_t add = (tid >= off) ? s_t[tid - off] : 0;
        __syncthreads();
        s_t[tid] += add;
        __syncthreads();
    }
    int64_t run = s_t[tid] - tot;   // exclusive prefix of this thread
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        if (base + u < n) data[base + u] = run;
        run += v[u];
    }
    if (sums && tid == kBlock - 1) sums[blockIdx.x] = s_t[kBlock - 1];
}

__global__ __launch_bounds__(kBlock) void k_add_chunk_prefix(int64_t* data, int64_t n, const int64_t* pre)
{
    const int64_t add = pre[blockIdx.x];
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanChunk;
    for (int j = threadIdx.x; j < kScanChunk; j += kBlock)
        if (base + j < n) data[base + j] += add;
}

template <typename RP>
__global__ __launch_bounds__(kBlock) void k_scatter_t(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                                      int64_t n_rows, unsigned long long* next,
                                                      int32_t* col_t, int64_t* perm)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= n_rows) return;
    const int64_t a = ld_rp(rp, i), e = ld_rp(rp, i + 1);
    for (int64_t kk = a; kk < e; ++kk) {
        const int64_t dst = static_cast<int64_t>(atomicAdd(next + col[kk], 1ull));
        col_t[dst] = static_cast<int32_t>(i);
        perm[dst] = kk;
    }
}

__global__ __launch_bounds__(kBlock) void k_sort_rows_t(const int64_t* __restrict__ rpt, int64_t n_cols,
                                                        int32_t* col_t, int64_t* perm)
{
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (j >= n_cols) return;
    const int64_t a = rpt[j], e = rpt[j + 1];
    for (int64_t m = a + 1; m < e; ++m) {   // insertion sort by original position
        const int64_t key = perm[m];
        const int32_t cv = col_t[m];
        int64_t h = m - 1;
        while (h >= a && perm[h] > key) {
            perm[h + 1] = perm[h];
            col_t[h + 1] = col_t[h];
            --h;
        }
        perm[h + 1] = key;
        col_t[h + 1] = cv;
    }
}

__global__ __launch_bounds__(kBlock) void k_narrow_i32(const int64_t* __restrict__ in, int32_t* out, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride)
        out[i] = static_cast<int32_t>(in[i]);
}

inline unsigned grid_for(int64_t n, int64_t per_block, int64_t cap = 65536)
{
    int64_t g = (n + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return static_cast<unsigned>(g);
}

hipError_t scan_exclusive(int64_t* data, int64_t n, int64_t* scratch, hipStream_t s)
{
    const int64_t nb = (n + kScanChunk - 1) / kScanChunk;
    if (nb <= 1) {
        hipLaunchKernelGGL(k_scan_chunks, dim3(1), dim3(kBlock), 0, s, data, n, static_cast<int64_t*>(nullptr));
        return hipGetLastError();
    }
    int64_t* sums = scratch;
    hipLaunchKernelGGL(k_scan_chunks, dim3(static_cast<unsigned>(nb)), dim3(kBlock), 0, s, data, n, sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = scan_exclusive(sums, nb, scratch + nb, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_add_chunk_prefix, dim3(static_cast<unsigned>(nb)), dim3(kBlock), 0, s, data, n,
                       static_cast<const int64_t*>(sums));
    return hipGetLastError();
}

template <typename RP>
hipError_t launch_spmv_rp(const CgArgs& a, int64_t k, int cap, hipStream_t s)
{
    const dim3 grid(a.G, a.batch), block(kBlock);
    if (cap <= kCapSmall) hipLaunchKernelGGL((k_cg_spmv<RP, kCapSmall>), grid, block, 0, s, a, k);
    else if (cap <= kCapMid) hipLaunchKernelGGL((k_cg_spmv<RP, kCapMid>), grid, block, 0, s, a, k);
    else hipLaunchKernelGGL((k_cg_spmv<RP, kCapLarge>), grid, block, 0, s, a, k);
    return hipGetLastError();
}

template <typename RP>
hipError_t launch_matvec_rp(const RP* rp, const int32_t* col, const double* vals, const double* x, double* y,
                            int64_t n_rows, int64_t nnz, int64_t n_cols, int batch, int cap, hipStream_t s)
{
    const int64_t ntiles = (n_rows + kTile - 1) / kTile;
    const dim3 grid(static_cast<unsigned>(ntiles), batch), block(kBlock);
    if (cap <= kCapSmall)
        hipLaunchKernelGGL((k_matvec<RP, kCapSmall>), grid, block, 0, s, rp, col, vals, x, y, n_rows, nnz, n_cols);
    else if (cap <= kCapMid)
        hipLaunchKernelGGL((k_matvec<RP, kCapMid>), grid, block, 0, s, rp, col, vals, x, y, n_rows, nnz, n_cols);
    else
        hipLaunchKernelGGL((k_matvec<RP, kCapLarge>), grid, block, 0, s, rp, col, vals, x, y, n_rows, nnz, n_cols);
    return hipGetLastError();
}

}  // namespace

// ----------------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------------
hipError_t launch_cg_init(const CgArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_init, dim3(a.G, a.batch), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_cg_spmv(const CgArgs& a, int64_t k, int rp_bits, int cap, hipStream_t s)
{
    return rp_bits == 64 ? launch_spmv_rp<int64_t>(a, k, cap, s) : launch_spmv_rp<int32_t>(a, k, cap, s);
}

hipError_t launch_cg_update(const CgArgs& a, int64_t k, hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_update, dim3(a.G, a.batch), dim3(kBlock), 0, s, a, k);
    return hipGetLastError();
}

hipError_t launch_matvec(const void* row_ptr, int rp_bits, const int32_t* col, const double* vals,
                         const double* x, double* y, int64_t n_rows, int64_t nnz, int64_t n_cols, int batch,
                         int cap, hipStream_t s)
{
    if (n_rows == 0) return hipSuccess;
    if (rp_bits == 64)
        return launch_matvec_rp(static_cast<const int64_t*>(row_ptr), col, vals, x, y, n_rows, nnz, n_cols, batch,
                                cap, s);
    return launch_matvec_rp(static_cast<const int32_t*>(row_ptr), col, vals, x, y, n_rows, nnz, n_cols, batch,
                            cap, s);
}

hipError_t launch_pattern_outer(const void* row_ptr, int rp_bits, const int32_t* col, double sign,
                                const double* u, int64_t us, const double* v, int64_t vs, double* g,
                                int64_t n_rows, int64_t nnz, int batch, hipStream_t s)
{
    if (n_rows == 0) return hipSuccess;
    const int64_t ntiles = (n_rows + kTile - 1) / kTile;
    const dim3 grid(static_cast<unsigned>(ntiles), batch), block(kBlock);
    if (rp_bits == 64)
        hipLaunchKernelGGL(k_pattern_outer<int64_t>, grid, block, 0, s, static_cast<const int64_t*>(row_ptr), col,
                           sign, u, us, v, vs, g, n_rows, nnz);
    else
        hipLaunchKernelGGL(k_pattern_outer<int32_t>, grid, block, 0, s, static_cast<const int32_t*>(row_ptr), col,
                           sign, u, us, v, vs, g, n_rows, nnz);
    return hipGetLastError();
}

hipError_t launch_gather_vals(const int64_t* perm, const double* vals, double* out, int64_t nnz, int batch,
                              hipStream_t s)
{
    if (nnz == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_vals, dim3(grid_for(nnz, kBlock, 4096), batch), dim3(kBlock), 0, s, perm, vals,
                       out, nnz);
    return hipGetLastError();
}

hipError_t launch_validate(const void* row_ptr, int rp_bits, const int32_t* col, int64_t n_rows, int64_t n_cols,
                           int64_t nnz, int32_t* err, int32_t* tile_max, hipStream_t s)
{
    const int64_t nb = n_rows / kBlock + 1;   // covers row n_rows's checks via i == 0 as well
    const dim3 grid(static_cast<unsigned>(nb)), block(kBlock);
    if (rp_bits == 64)
        hipLaunchKernelGGL(k_validate<int64_t>, grid, block, 0, s, static_cast<const int64_t*>(row_ptr), col, n_rows,
                           n_cols, nnz, err, tile_max);
    else
        hipLaunchKernelGGL(k_validate<int32_t>, grid, block, 0, s, static_cast<const int32_t*>(row_ptr), col, n_rows,
                           n_cols, nnz, err, tile_max);
    return hipGetLastError();
}

size_t transpose_scratch_bytes(int64_t n_rows, int64_t n_cols, int64_t nnz)
{
    (void)n_rows;
    (void)nnz;
    // counts/row pointers (n_cols + 1), cursors (n_cols + 1), scan partial sums
    int64_t levels = 0, m = n_cols + 1;
    while (m > 1) {
        m = (m + kScanChunk - 1) / kScanChunk;
        levels += m + 1;
    }
    return static_cast<size_t>(2 * (n_cols + 1) + levels + 16) * sizeof(int64_t);
}

hipError_t launch_transpose(const void* row_ptr, int rp_bits, const int32_t* col, int64_t n_rows, int64_t n_cols,
                            int64_t nnz, void* row_ptr_t, int32_t* col_t, int64_t* perm, void* scratch,
                            hipStream_t s)
{
    int64_t* cnt = static_cast<int64_t*>(scratch);    // -> row pointers of A^T (int64)
    int64_t* next = cnt + (n_cols + 1);                // scatter cursors
    int64_t* sums = next + (n_cols + 1);
    hipLaunchKernelGGL(k_fill_i64, dim3(grid_for(n_cols + 1, kBlock, 4096)), dim3(kBlock), 0, s, cnt, n_cols + 1,
                       static_cast<int64_t>(0));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nnz > 0) {
        hipLaunchKernelGGL(k_count_cols, dim3(grid_for(nnz, kBlock, 8192)), dim3(kBlock), 0, s, col, nnz,
                           reinterpret_cast<unsigned long long*>(cnt));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = scan_exclusive(cnt, n_cols + 1, sums, s)) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(next, cnt, sizeof(int64_t) * (n_cols + 1), hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return e;
    if (n_rows > 0 && nnz > 0) {
        const dim3 grid(grid_for(n_rows, kBlock, INT32_MAX)), block(kBlock);
        if (rp_bits == 64)
            hipLaunchKernelGGL(k_scatter_t<int64_t>, grid, block, 0, s, static_cast<const int64_t*>(row_ptr), col,
                               n_rows, reinterpret_cast<unsigned long long*>(next), col_t, perm);
        else
            hipLaunchKernelGGL(k_scatter_t<int32_t>, grid, block, 0, s, static_cast<const int32_t*>(row_ptr), col,
                               n_rows, reinterpret_cast<unsigned long long*>(next), col_t, perm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (n_cols > 0 && nnz > 0) {
        hipLaunchKernelGGL(k_sort_rows_t, dim3(grid_for(n_cols, kBlock, INT32_MAX)), dim3(kBlock), 0, s,
                           static_cast<const int64_t*>(cnt), n_cols, col_t, perm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (rp_bits == 64)
        return hipMemcpyAsync(row_ptr_t, cnt, sizeof(int64_t) * (n_cols + 1), hipMemcpyDeviceToDevice, s);
    hipLaunchKernelGGL(k_narrow_i32, dim3(grid_for(n_cols + 1, kBlock, 4096)), dim3(kBlock), 0, s,
                       static_cast<const int64_t*>(cnt), static_cast<int32_t*>(row_ptr_t), n_cols + 1);
    return hipGetLastError();
}

}  // namespace sla
