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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "sla_internal.h"

namespace sla {

LaunchEvents& launch_events()
{
    static thread_local LaunchEvents ev;
    return ev;
}

// Launch through hipExtLaunchKernelGGL when timing events are armed for this launch.
#define SLA_LAUNCH(kernel, grid, block, shmem, stream, ...)                                          \
    do {                                                                                             \
        LaunchEvents& le_ = launch_events();                                                         \
        if (le_.start)                                                                               \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, le_.start, le_.stop, 0,        \
                                  __VA_ARGS__);                                                      \
        else                                                                                         \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                     \
    } while (0)

namespace {

// Gathers kept in flight per row: the variant for <= 5 entries per row on average
// takes 5 (one round for 5-point stencils), the wider variants 8.
constexpr int row_chunk(int cap) { return cap <= kCapSmall ? 5 : 8; }

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

// Deterministic sum of G partials written by the previous kernel: thread t adds
// part[t], part[t + kBlock], ... in that order, then the fixed workgroup tree.  The
// loads of a trip of 8 (G <= 2048 in one trip) are all issued before the first is
// added, so the reduction costs one memory round trip rather than one per partial.
__device__ __forceinline__ double reduce_partials(const double* part, int G, double* s_red)
{
    constexpr int U = 8;
    double v = 0.0;
    for (int i0 = threadIdx.x; i0 < G; i0 += U * kBlock) {
        double t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) t[u] = part[min(i0 + u * kBlock, G - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) v = (i0 + u * kBlock < G) ? v + t[u] : v;
    }
    return block_sum(v, s_red);
}

// Tiles of one workgroup.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup b runs on XCD b % 8).  With the XCD mapping each XCD owns one contiguous
// eighth [lo, lo + len) of the tiles, and its G/8 workgroups take the positions
// first, first + step, ... < len of that range, so they sweep through it together.
struct TileRange {
    int64_t lo, len, first, step;
};

__device__ __forceinline__ TileRange tile_range(int G, int64_t ntiles, int remap)
{
    const int bx = blockIdx.x;
    if (remap && (G & 7) == 0 && G >= 16) {
        const int x = bx & 7;
        const int64_t lo = (ntiles * x) >> 3;
        const int64_t hi = (ntiles * (x + 1)) >> 3;
        return TileRange{lo, hi - lo, bx >> 3, G >> 3};
    }
    return TileRange{0, ntiles, bx, G};
}

// Which system and which of its workgroups this is, and its tiles.  For batches of
// 8 or more systems (batch % 8 == 0) the grid is read as one linear sequence and
// every system is pinned to one XCD: XCD x runs systems x, x + 8, x + 16, ... one
// after the other, all G workgroups of a system on that XCD.  The gathered vectors of
// the systems in flight then stay in that XCD's L2 instead of being spread over all
// eight (each XCD would otherwise hold a slice of every running system).
struct BlockCoord {
    int sys;
    int lb;      // workgroup index within the system: its partial-sum slot
    TileRange tr;
};

__device__ __forceinline__ BlockCoord block_coord(const CgArgs& a, int G)
{
    if (a.list_wg) {
        // SparseTensorList: system of workgroup L by binary search in the workgroup table
        const int64_t L = blockIdx.x;
        int lo = 0, hi = a.list_items;   // list_wg[lo] <= L < list_wg[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.list_wg[mid] <= L) lo = mid;
            else hi = mid;
        }
        const int32_t g0 = a.list_wg[lo], gi = a.list_wg[lo + 1] - g0;
        const int64_t t0 = a.list_tiles[lo], len = a.list_tiles[lo + 1] - t0;
        const int j = static_cast<int>(L - g0);
        if ((gi & 7) == 0) {
            // the item's workgroups j, j + 8, ... run on one XCD (workgroup L on XCD L % 8):
            // they sweep one contiguous eighth of the item's tiles, so the neighbouring
            // tiles a tile's rows reach into are read through that XCD's L2
            const int x = j & 7;
            const int64_t tlo = (len * x) >> 3, thi = (len * (x + 1)) >> 3;
            return BlockCoord{lo, j, TileRange{t0 + tlo, thi - tlo, j >> 3, gi >> 3}};
        }
        return BlockCoord{lo, j, TileRange{t0, len, j, gi}};
    }
    if (a.sys_per_xcd) {
        const int64_t L = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
        const int x = static_cast<int>(L & 7);
        const int64_t slot = L >> 3;
        const int sys = x + 8 * static_cast<int>(slot / G);
        const int lb = static_cast<int>(slot % G);
        return BlockCoord{sys, lb, TileRange{0, a.ntiles, lb, G}};
    }
    return BlockCoord{static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.x),
                      tile_range(G, a.ntiles, a.xcd_remap)};
}

// Partial-sum slots of system sys when each system has G workgroups (a table in list
// mode), and the offsets of its vectors and values.
struct Parts {
    int64_t base;
    int count;
};
__device__ __forceinline__ Parts parts_of(const CgArgs& a, int sys, int G)
{
    if (a.list_wg) {
        const int64_t lo = a.list_wg[sys];
        return Parts{lo, static_cast<int>(a.list_wg[sys + 1] - lo)};
    }
    return Parts{static_cast<int64_t>(sys) * G, G};
}
__device__ __forceinline__ int64_t vec_off(const CgArgs& a, int sys)
{
    return a.list_wg ? 0 : static_cast<int64_t>(sys) * a.n;
}
__device__ __forceinline__ int64_t val_off(const CgArgs& a, int sys)
{
    return a.list_wg ? 0 : static_cast<int64_t>(sys) * a.nnz;
}
__device__ __forceinline__ double reduce_parts(const double* part, Parts p, double* s_red)
{
    return reduce_partials(part + p.base, p.count, s_red);
}

template <typename RP>
__device__ __forceinline__ int64_t ld_rp(const RP* rp, int64_t i)
{
    return static_cast<int64_t>(rp[i]);
}

// Row pointer at a workgroup-uniform index, read through the constant address space
// so it becomes a scalar load: its wait counts on the scalar counter and does not
// drain the vector loads in flight.  The row pointers are never written by a kernel.
template <typename RP>
__device__ __forceinline__ int64_t ld_rp_uniform(const RP* rp, int64_t i)
{
    typedef const __attribute__((address_space(4))) RP* cptr;
    return static_cast<int64_t>(((cptr)(rp))[i]);
}

// Element c of a vector.  With OFF32 (vectors shorter than 2^29 entries) the address
// is a uniform 64-bit base plus a 32-bit byte offset, which the compiler maps to one
// VGPR per gather instead of a 64-bit address pair.
template <bool OFF32>
__device__ __forceinline__ double ldv(const double* __restrict__ base, int64_t c)
{
    if constexpr (OFF32)
        return *reinterpret_cast<const double*>(reinterpret_cast<const char*>(base) +
                                                (static_cast<uint32_t>(c) << 3));
    else
        return base[c];
}

// Gathered operand of the CG SpMV: p_k[c] = r_k[c] + beta * p_{k-1}[c].  For k = 0,
// r_0 = b, beta = 0 and p_{-1} = 0 (zeroed by k_cg_init), which gives p_0 = b exactly.
template <bool OFF32>
struct GatherCG {
    const double* __restrict__ rin;
    const double* __restrict__ pprev;
    double beta;
    __device__ __forceinline__ double operator()(int64_t c) const
    {
        const double rv = ldv<OFF32>(rin, c);
        const double t = beta * ldv<OFF32>(pprev, c);
        return rv + t;
    }
};

template <bool OFF32>
struct GatherX {
    const double* __restrict__ x;
    __device__ __forceinline__ double operator()(int64_t c) const { return ldv<OFF32>(x, c); }
};

// Row-length bins of a tile whose entries exceed the LDS cap.
constexpr int kBinLaneMax = 32;     // rows of at most this many entries: one lane per row
constexpr int kBinGroupMax = 512;   // then one 16-lane group per row; longer rows: the workgroup
constexpr int kBinGroup = 16;
// Gathers in flight per lane in the group and workgroup bins.  Those bins sit in every
// capped SpMV, and a kernel's registers are those of its widest path: at 8 they took
// the BiCGStab products from 110 to 131 VGPRs (4 to 3 waves per SIMD, 15.9 to 18.3 us
// at 1M rows).  A row of more than kBinLaneMax entries sends its pattern to the
// products-first kernels, so in the capped kernels these bins only guard.
constexpr int kBinUnroll = 4;

// Sum over a 16-lane group (lanes of one group only), fixed xor tree.
__device__ __forceinline__ double group16_sum(double v)
{
#pragma unroll
    for (int off = kBinGroup / 2; off > 0; off >>= 1) v = v + __shfl_xor(v, off, kBinGroup);
    return v;
}

// This lane's share of a row: entries ra + lane0, ra + lane0 + stride, ... < re, summed
// in that order, kBinUnroll gathers in flight (clamped addresses, masked sums).
template <typename RP, typename G>
__device__ __forceinline__ double strided_rowpart(const int32_t* __restrict__ col, const double* __restrict__ vals,
                                                  int64_t ra, int64_t re, int lane0, int stride, const G& g)
{
    double acc = 0.0;
    for (int64_t k0 = ra + lane0; k0 < re; k0 += static_cast<int64_t>(stride) * kBinUnroll) {
        double v[kBinUnroll], p[kBinUnroll];
#pragma unroll
        for (int u = 0; u < kBinUnroll; ++u) {
            const int64_t k = k0 + static_cast<int64_t>(u) * stride;
            const int64_t j = k < re ? k : k0;
            v[u] = vals[j];
            p[u] = g(col[j]);
        }
#pragma unroll
        for (int u = 0; u < kBinUnroll; ++u) {
            const bool ok = k0 + static_cast<int64_t>(u) * stride < re;
            const double t = v[u] * p[u];
            const double an = acc + t;
            acc = ok ? an : acc;
        }
    }
    return acc;
}

// Row sums of a tile whose entries exceed the LDS cap, binned by row length (the rows
// are read from global memory, not staged):
//   * at most kBinLaneMax entries: the row's own lane sums it sequentially in ascending
//     entry order, RC gathers in flight -- the oracle's order, so these rows are exact;
//   * up to kBinGroupMax: a 16-lane group per row (four rows per wave at a time), each
//     lane summing the entries j = lane, lane + 16, ... of the row in order, then a
//     fixed xor tree over the group;
//   * longer rows: the whole workgroup per row, one after the other, each thread summing
//     the entries j = tid, tid + 256, ... in order, then the fixed workgroup tree.
// Group and workgroup rows are listed in LDS (s_col) by an atomic append: which group
// takes a row varies, but each row's sum does not.  Every thread of the workgroup must
// call it (workgroup barriers); s_val holds kTile doubles, s_col kTile + 2 ints.
template <typename RP, int RC, typename G>
__device__ __forceinline__ double tile_rowsum_long(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                                const double* __restrict__ vals, int64_t row0, int nr,
                                                const G& g, double* s_val, int32_t* s_col)
{
    __shared__ double s_red[kBlock / 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    int32_t* s_list = s_col;              // [0, n_grp): group rows; from the top down: workgroup rows
    int32_t* s_cnt = s_col + kTile;       // [0] group rows, [1] workgroup rows
    double* s_q = s_val;
    if (tid < 2) s_cnt[tid] = 0;
    __syncthreads();
    const int tl = min(tid, nr - 1);
    const int64_t a = ld_rp(rp, row0 + tl);
    const int64_t e = (tid < nr) ? ld_rp(rp, row0 + tl + 1) : a;
    const int64_t len = e - a;
    double s = 0.0;
    if (len > kBinLaneMax) {
        if (len > kBinGroupMax) s_list[kTile - 1 - atomicAdd(&s_cnt[1], 1)] = tid;
        else s_list[atomicAdd(&s_cnt[0], 1)] = tid;
    } else {
        for (int64_t j0 = a; j0 < e; j0 += RC) {
            double pv[RC], vv[RC];
#pragma unroll
            for (int u = 0; u < RC; ++u) {
                const int64_t j = (j0 + u < e) ? j0 + u : j0;
                vv[u] = vals[j];
                pv[u] = g(col[j]);
            }
#pragma unroll
            for (int u = 0; u < RC; ++u) {
                const bool ok = j0 + u < e;
                const double t = vv[u] * pv[u];
                const double sn = s + t;
                s = ok ? sn : s;
            }
        }
    }
    __syncthreads();
    const int n_grp = s_cnt[0], n_wg = s_cnt[1];
    // 16-lane groups: group gi of the workgroup takes rows gi, gi + 16, ... of the list
    const int sub = lane & (kBinGroup - 1);
    const int gi = tid / kBinGroup;
    constexpr int kGroups = kBlock / kBinGroup;
    for (int base = 0; base < n_grp; base += kGroups) {   // uniform trip count
        const int li = base + gi;
        const int rr = li < n_grp ? s_list[li] : -1;
        double acc = 0.0;
        if (rr >= 0) acc = strided_rowpart<RP>(col, vals, ld_rp(rp, row0 + rr), ld_rp(rp, row0 + rr + 1), sub,
                                               kBinGroup, g);
        acc = group16_sum(acc);
        if (rr >= 0 && sub == 0) s_q[rr] = acc;
    }
    // the longest rows: the whole workgroup on each
    for (int wi = 0; wi < n_wg; ++wi) {
        const int rr = s_list[kTile - 1 - wi];
        double acc = strided_rowpart<RP>(col, vals, ld_rp(rp, row0 + rr), ld_rp(rp, row0 + rr + 1), tid, kBlock, g);
        acc = block_sum(acc, s_red);
        if (tid == 0) s_q[rr] = acc;
    }
    __syncthreads();
    if (len > kBinLaneMax) s = s_q[tid];
    __syncthreads();
    return (tid < nr) ? s : 0.0;
}

// Rows of more than this many entries are summed by the workgroup in the
// products-first kernels (a fixed tree); shorter ones by their own lane, in order.
constexpr int kBinSeqMax = 1024;

// Row sums of one tile, products first (patterns with a row of more than kBinLaneMax
// entries).  The tile's entries go through LDS in chunks of kCapLarge: per chunk every
// thread forms the products of entries j = tid, tid + kBlock, ... (values and columns
// loaded coalesced, all gathers in flight at once, spread evenly whatever the row
// lengths) and stores them; then each lane adds its row's products of the chunk in
// ascending order, carrying its sum across chunks.  The products are the rounded
// val * x[col] and the order ascending, so rows of up to kBinSeqMax entries get the
// oracle's sums to the bit; longer rows are summed by the whole workgroup (each
// thread's strided share in order, then the fixed tree).  Every thread of the
// workgroup must call it (workgroup barriers); s_val holds kCapLarge doubles, s_col
// kTile + 2 ints.
template <typename RP, typename G>
__device__ __forceinline__ double tile_rowsum_pf(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                              const double* __restrict__ vals, int64_t row0, int nr, const G& g,
                                              double* s_val, int32_t* s_col)
{
    __shared__ double s_red[kBlock / 64];
    constexpr int C = kCapLarge;
    constexpr int U = C / kBlock;
    const int tid = threadIdx.x;
    const int64_t k0 = ld_rp(rp, row0);
    const int64_t cnt = ld_rp(rp, row0 + nr) - k0;
    const int tl = min(tid, nr - 1);
    const int64_t rs = ld_rp(rp, row0 + tl) - k0;
    const int64_t re = (tid < nr) ? ld_rp(rp, row0 + tl + 1) - k0 : rs;
    const bool lng = re - rs > kBinSeqMax;
    double s = 0.0;
    for (int64_t c0 = 0; c0 < cnt; c0 += C) {   // uniform trip count
        const int clen = static_cast<int>(min(static_cast<int64_t>(C), cnt - c0));
        const double* __restrict__ vb = vals + k0 + c0;
        const int32_t* __restrict__ cb = col + k0 + c0;
        double v[U], pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(tid + u * kBlock, clen - 1);
            v[u] = vb[j];
            pv[u] = g(cb[j]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = tid + u * kBlock;
            if (j < clen) s_val[j] = v[u] * pv[u];
        }
        __syncthreads();
        if (!lng) {
            const int a0 = static_cast<int>(max(rs - c0, int64_t(0)));
            const int a1 = static_cast<int>(min(re - c0, static_cast<int64_t>(clen)));
#pragma unroll 4
            for (int j = a0; j < a1; ++j) s = s + s_val[j];
        }
        __syncthreads();
    }
    if (__syncthreads_or(lng)) {
        int32_t* s_list = s_col;
        int32_t* s_cnt = s_col + kTile;
        if (tid == 0) s_cnt[0] = 0;
        __syncthreads();
        if (lng) s_list[atomicAdd(&s_cnt[0], 1)] = tid;
        __syncthreads();
        const int n_long = s_cnt[0];
        for (int wi = 0; wi < n_long; ++wi) {
            const int rr = s_list[wi];
            double acc = strided_rowpart<RP>(col, vals, ld_rp(rp, row0 + rr), ld_rp(rp, row0 + rr + 1), tid, kBlock, g);
            acc = block_sum(acc, s_red);
            if (tid == 0) s_val[rr] = acc;
        }
        __syncthreads();
        if (lng) s = s_val[tid];
        __syncthreads();
    }
    return (tid < nr) ? s : 0.0;
}

// Row sums of one tile [row0, row0 + nr) for lane tid (0 for tid >= nr).  Contains
// the workgroup barriers of the LDS staging; every thread of the workgroup must call it.
// Loads are never behind a divergent branch: out-of-range slots re-read a valid
// address (clamped index) and their contribution is masked, so all loads of a phase
// are in flight together instead of one memory round trip per entry.
template <typename RP, int CAP, int RC, typename G>
__device__ __forceinline__ double tile_rowsum(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                              const double* __restrict__ vals, int64_t row0, int nr,
                                              const G& g, double* s_val, int32_t* s_col)
{
    if constexpr (CAP == kCapSkew) return tile_rowsum_pf<RP>(rp, col, vals, row0, nr, g, s_val, s_col);
    const int tid = threadIdx.x;
    const int64_t k0 = ld_rp(rp, row0);
    const int64_t k1 = ld_rp(rp, row0 + nr);
    const int64_t cnt = k1 - k0;
    double s = 0.0;
    if (cnt <= CAP) {
        const int tl = min(tid, nr - 1);
        const int rs = static_cast<int>(ld_rp(rp, row0 + tl) - k0);
        const int re = (tid < nr) ? static_cast<int>(ld_rp(rp, row0 + tl + 1) - k0) : rs;
        if (cnt > 0) {
            constexpr int U = CAP / kBlock;
            const double* __restrict__ vb = vals + k0;
            const int32_t* __restrict__ cb = col + k0;
            const int last = static_cast<int>(cnt) - 1;
            double v[U];
            int32_t c[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = min(tid + u * kBlock, last);
                v[u] = vb[j];
                c[u] = cb[j];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = tid + u * kBlock;
                if (j < cnt) {
                    s_val[j] = v[u];
                    s_col[j] = c[u];
                }
            }
        }
        __syncthreads();
        for (int j0 = rs; j0 < re; j0 += RC) {
            double pv[RC];
#pragma unroll
            for (int u = 0; u < RC; ++u) {
                const int j = (j0 + u < re) ? j0 + u : j0;
                pv[u] = g(s_col[j]);
            }
#pragma unroll
            for (int u = 0; u < RC; ++u) {
                const bool ok = j0 + u < re;
                const int j = ok ? j0 + u : j0;
                const double t = s_val[j] * pv[u];
                const double sn = s + t;
                s = ok ? sn : s;
            }
        }
        __syncthreads();
    } else {
        s = tile_rowsum_long<RP, RC>(rp, col, vals, row0, nr, g, s_val, s_col);
    }
    return s;
}

// ----------------------------------------------------------------------------------
// CG kernels.  Grid: (G, batch) workgroups of kBlock threads; workgroup b of system
// `sys` owns the tiles of tile_range(); it writes partial sums into slot b.
// ----------------------------------------------------------------------------------
constexpr int kStreamUnroll = 4;   // tiles per loop trip of the streaming kernels

// Jacobi: k_cg_diag stores one flag per workgroup, kDiagNaN if some diagonal entry of
// its rows is NaN, else kDiagNonPos if one is <= 0 or missing, else 0.  Summed over
// the (at most 65535) workgroups of a system, the total reaches kDiagNaN exactly when
// some entry is NaN.
constexpr double kDiagNonPos = 1.0;
constexpr double kDiagNaN = 65536.0;

__global__ __launch_bounds__(kBlock) void k_cg_init(CgArgs a)
{
    __shared__ double s_red[kBlock / 64];
    const BlockCoord bc = block_coord(a, a.Gu);
    const int sys = bc.sys;
    const int tid = threadIdx.x;
    const int lb = bc.lb;
    const TileRange tr = bc.tr;
    const int64_t off = vec_off(a, sys);
    const double* __restrict__ b = a.b + off;
    double* __restrict__ x = a.x + off;
    double* __restrict__ pm1 = a.p1 + off;   // p_{-1} = 0
    const bool jac = a.jacobi != 0;
    double rr = 0.0, rz = 0.0;
    for (int64_t m0 = tr.first; m0 < tr.len; m0 += kStreamUnroll * tr.step) {
        double bv[kStreamUnroll], dv[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t i = min((tr.lo + m0 + u * tr.step) * kTile + tid, a.n - 1);
            bv[u] = b[i];
            dv[u] = jac ? a.dg[off + i] : 1.0;
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t m = m0 + u * tr.step;
            const int64_t i = (tr.lo + m) * kTile + tid;
            if (m < tr.len && i < a.n) {
                x[i] = 0.0;
                pm1[i] = 0.0;
                const double w = bv[u] * bv[u];
                rr = rr + w;
                if (jac) {                       // z_0 = M^{-1} b
                    const double zv = bv[u] / dv[u];
                    a.z[off + i] = zv;
                    const double wz = bv[u] * zv;
                    rz = rz + wz;
                }
            }
        }
    }
    rr = block_sum(rr, s_red);
    if (jac) rz = block_sum(rz, s_red);
    const int64_t slot = parts_of(a, sys, a.Gu).base + lb;
    if (tid == 0) {
        if (jac) {
            a.part_rr[slot] = rr;
            a.part_rho[slot] = rz;
        } else {
            a.part_rho[slot] = rr;
        }
        if (lb == 0) a.st[sys].stop_iter = INT64_MAX;
        if (lb == 0 && sys == 0) *a.n_active = a.list_wg ? a.list_items : a.batch;
    }
}

__device__ __forceinline__ double block_max(double v, double* s_red)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s_red[w] = v;
    __syncthreads();
    const double t = fmax(fmax(s_red[0], s_red[1]), fmax(s_red[2], s_red[3]));
    __syncthreads();
    return t;
}

// Jacobi: the diagonal of A (entry (i, i) found by binary search in the ascending
// columns of row i; 0 if not stored) into dg, and the workgroup's flag partial (see
// kDiagNaN).  Same grid and partial slots as k_cg_init, which runs after it.
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_cg_diag(CgArgs a)
{
    __shared__ double s_red[kBlock / 64];
    const BlockCoord bc = block_coord(a, a.Gu);
    const int sys = bc.sys;
    const int tid = threadIdx.x;
    const TileRange tr = bc.tr;
    const RP* __restrict__ rp = static_cast<const RP*>(a.row_ptr);
    const double* __restrict__ vals = a.vals + val_off(a, sys);
    double* __restrict__ dg = a.dg + vec_off(a, sys);
    // list mode: the padding rows of the system's last tile take d = 1 (r = 0 there)
    const int64_t rend = a.list_wg ? a.list_rend[sys] : a.n;
    double flag = 0.0;
    for (int64_t m = tr.first; m < tr.len; m += tr.step) {
        const int64_t i = (tr.lo + m) * kTile + tid;
        if (i >= rend && i < a.n) dg[i] = 1.0;
        if (i < rend) {
            int64_t lo = ld_rp(rp, i), hi = ld_rp(rp, i + 1);
            while (lo < hi) {
                const int64_t mid = (lo + hi) >> 1;
                if (a.col[mid] < i) lo = mid + 1;
                else hi = mid;
            }
            const double d = (lo < ld_rp(rp, i + 1) && a.col[lo] == i) ? vals[lo] : 0.0;
            dg[i] = d;
            if (d != d) flag = kDiagNaN;
            else if (!(d > 0.0)) flag = fmax(flag, kDiagNonPos);
        }
    }
    flag = block_max(flag, s_red);
    if (tid == 0) a.part_aux[parts_of(a, sys, a.Gu).base + bc.lb] = flag;
}

// Start of a CG SpMV launch for system sys at iteration k: read the stop word, sum
// the rho partials (rho_k = r_k^T r_k), and decide.  Returns kStepStopped if the
// system stopped in an earlier launch, kStepStopNow if it stops at k (the info record
// and the stop word are written here; the caller applies the deferred x update), else
// kStepRun with beta_k = rho_k / rho_{k-1} (0 for k = 0) and alpha_{k-1} (0 for
// k = 0).  Contains workgroup barriers: every thread of the workgroup calls it.
constexpr int kStepRun = 0;
constexpr int kStepStopped = 1;
constexpr int kStepStopNow = 2;

// Variants of the staged SpMV kernel k_cg_spmv.
constexpr int kSpmvFused = 0;   // CG, p_k formed on the fly, deferred x update
constexpr int kSpmvSplit = 1;   // CG, split schedule: p_k read as formed
constexpr int kSpmvBsV = 2;     // BiCGStab: v = A p, partial <rh, v>
constexpr int kSpmvBsT = 3;     // BiCGStab: t = A s, partials <t, s>, <t, t>

// BiCGStab's kernels of iteration k run in the order p update, v = A p, s, t = A s,
// update; the stop word of a system holds the phase (5 k + position) of the kernel
// that stopped it.  A kernel returns at once if the word is below its own phase; the
// workgroups of the deciding kernel, which may read the word their leader just wrote,
// see it equal to their phase and take the same decision again.
constexpr int kPhaseP = 0, kPhaseV = 1, kPhaseS = 2, kPhaseT = 3, kPhaseU = 4;
__device__ __forceinline__ int64_t bs_phase(int64_t k, int pos) { return 5 * k + pos; }

// The vector p_k is formed from: r_k (r_0 = b, never copied) or, with Jacobi, z_k.
__device__ __forceinline__ const double* gathered_r(const CgArgs& a, bool first)
{
    return a.jacobi ? a.z : (first ? a.b : a.r);
}


__device__ __forceinline__ int cg_step_begin(const CgArgs& a, int sys, int lb, int64_t k, double* s_red,
                                             int64_t* s_stop, double& beta, double& alpha_prev)
{
    SysState* st = a.st + sys;
    const int tid = threadIdx.x;
    const bool lead = (lb == 0 && tid == 0);
    const bool first = (k == 0);
    // One read of the stop word per workgroup (published by the barriers of the
    // reduction), so the exit decision is uniform even while this kernel's leading
    // workgroup may be writing stop_iter = k.
    if (tid == 0) *s_stop = st->stop_iter;
    const Parts pu = parts_of(a, sys, a.Gu);
    const double rho_k = reduce_parts(a.part_rho, pu, s_red);
    // |r_k|: from rho_k itself, or (Jacobi, rho_k = r^T z) from its own partials
    const double rr_k =
        a.jacobi ? reduce_parts(a.part_rr, pu, s_red) : rho_k;
    const double diag_flags =
        (a.jacobi && first) ? reduce_parts(a.part_aux, pu, s_red) : 0.0;
    beta = 0.0;
    alpha_prev = 0.0;
    if (*s_stop < k) return kStepStopped;
    const double res = sqrt(rr_k);
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
    alpha_prev = first ? 0.0 : st->alpha[(k - 1) & 1];

    int code = -1;
    if (!a.fixed && res <= thr) code = SLA_CONVERGED;
    else if (diag_flags >= kDiagNaN) code = SLA_NAN;        // Jacobi, k = 0: unusable diagonal
    else if (diag_flags > 0.0) code = SLA_NOT_SPD;
    else if (k >= a.max_iter) code = SLA_MAX_ITER;
    if (code >= 0) {
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
        return kStepStopNow;
    }
    beta = first ? 0.0 : rho_k / st->rho[(k - 1) & 1];
    if (lead) {
        st->rho[k & 1] = rho_k;
        st->rr = rr_k;
        if (first) { st->thr = thr; st->rhs = rhs; }
    }
    return kStepRun;
}

// Staged data of one tile, held in registers until the tile is processed: its
// entries (written to LDS then), this lane's row bounds, and this lane's row of the
// vectors the update needs.  Nothing derived from these loads is computed at staging
// time, so no wait is forced until the tile is consumed.
template <typename RP, int U>
struct TileStage {
    double v[U];
    int32_t c[U];
    RP a0, a1;            // row_ptr[row], row_ptr[row + 1] of this lane's (clamped) row
    double ri, ppi, xi;   // r_k, p_{k-1}, x_{k-1} at this lane's row
};

// Issue (without waiting) the loads of tile t.  k0 / k1 are the tile's first and
// end entry positions (known two tiles ahead).  Indices are clamped so no load sits
// behind a branch; the tile's entries are staged only if they fit the LDS cap.
// C16: the columns are read from the 16-bit offsets col16 (column minus the tile's
// first row, sign-extended by the load itself); the tile's first row is added when
// they are written to LDS.
template <typename RP, int CAP, bool OFF32, bool SPLIT, bool C16>
__device__ __forceinline__ void stage_tile(TileStage<RP, CAP / kBlock>& S, const RP* __restrict__ rp,
                                           const int32_t* __restrict__ col, const int16_t* __restrict__ col16,
                                           const double* __restrict__ vals,
                                           const double* __restrict__ rin, const double* __restrict__ pprev,
                                           const double* __restrict__ x, int64_t t, int64_t n, int64_t k0,
                                           int64_t k1, bool live = true)
{
    constexpr int U = CAP / kBlock;
    const int tid = threadIdx.x;
    const int64_t row0 = t * kTile;
    const int nr = static_cast<int>(min(static_cast<int64_t>(kTile), n - row0));
    // live = false: a stand-in stage past the workgroup's last tile (loads issued, never
    // used), every lane at the tile's first row and (k0 = k1) its first entry, so it
    // costs a few cache lines
    const int64_t i = row0 + (live ? min(tid, nr - 1) : 0);
    S.a0 = rp[i];
    S.a1 = rp[i + 1];
    S.ri = ldv<OFF32>(rin, i);   // with SPLIT: p_k (rin is the formed operand)
    if constexpr (!SPLIT) {
        S.ppi = ldv<OFF32>(pprev, i);
        S.xi = x[i];
    }
    const int64_t cnt = k1 - k0;
    // (the products-first variant reads its entries itself, chunk by chunk)
    // Unconditional: an empty or over-cap tile loads clamped copies of stored entries
    // (never read), so every staged register is written on every path and no load in
    // flight is drained where paths join.  (A pattern with no stored entries gets
    // readable stand-in pointers from the host.)
    if constexpr (CAP != kCapSkew) {
        const int64_t kb = cnt > 0 ? k0 : (k0 > 0 ? k0 - 1 : 0);
        const double* __restrict__ vb = vals + kb;
        const int last = static_cast<int>(min(max(cnt, static_cast<int64_t>(1)), static_cast<int64_t>(CAP))) - 1;
        if constexpr (C16) {
            const int16_t* __restrict__ cb = col16 + kb;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = min(tid + u * kBlock, last);
                S.v[u] = vb[j];
                S.c[u] = cb[j];
            }
        } else {
            const int32_t* __restrict__ cb = col + kb;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = min(tid + u * kBlock, last);
                S.v[u] = vb[j];
                S.c[u] = cb[j];
            }
        }
    }
}

// k_cg_spmv: one CG iteration's SpMV with everything fused around it.  Tiles are
// software-pipelined: while the gathers of tile t are in flight, the row pointers
// and entries of the workgroup's next tile are already loading (and the bounds of
// the one after), so each tile costs about one memory round trip instead of four.
// The first tile is staged before the stop check and the reduction of the rho
// partials, which overlaps the kernel's start-up latency with useful loads.
//
// MODE kSpmvSplit: the split schedule for unstructured patterns.  k_cg_pupd has
// already taken the step's decisions and formed p_k (and the x update); this kernel
// gathers p_k alone, one load per stored entry instead of two (r_k and p_{k-1}), and
// computes q and the partial p^T q.  The row sums are the same to the last bit.
// MODE kSpmvBsV / kSpmvBsT: the two products of a BiCGStab iteration, v = A p with
// the partial <rh, v> (rh = b), and t = A s with the partials <t, s> and <t, t>.
//
// C16: the staged columns come from the 16-bit tile offsets a.col16 (2 bytes per entry
// instead of 4); tiles past the LDS cap still read the 32-bit columns.
template <typename RP, int CAP, bool OFF32, int MODE, bool C16>
__global__ __launch_bounds__(kBlock) void k_cg_spmv(CgArgs a, int64_t k)
{
    constexpr bool SPLIT = MODE != kSpmvFused;
    constexpr int U = CAP / kBlock;
    constexpr int RC = row_chunk(CAP);
    __shared__ double s_val[CAP];
    __shared__ int32_t s_col[CAP];
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const BlockCoord bc = block_coord(a, a.G);
    const int sys = bc.sys;
    const int tid = threadIdx.x;
    const int lb = bc.lb;
    const TileRange tr = bc.tr;
    const bool first = (k == 0);
    const int64_t off = vec_off(a, sys);
    const int64_t n = a.n;
    const RP* __restrict__ rp = static_cast<const RP*>(a.row_ptr);
    const int32_t* __restrict__ col = a.col;
    const int16_t* __restrict__ col16 = a.col16;
    const double* __restrict__ vals = a.vals + val_off(a, sys);
    const int64_t ntiles = tr.len;   // positions of this workgroup: tr.first + j * step, below tr.len
    const int64_t Gs = tr.step;
    auto tile_of = [&](int64_t m) { return tr.lo + m; };
    auto tile_k0 = [&](int64_t m) { return ld_rp_uniform(rp, tile_of(m) * kTile); };
    auto tile_k1 = [&](int64_t m) { return ld_rp_uniform(rp, min((tile_of(m) + 1) * kTile, n)); };
    const double* __restrict__ rin = gathered_r(a, first) + off;         // r_k (r_0 = b), or z_k
    const double* __restrict__ pprev = ((k & 1) ? a.p0 : a.p1) + off;   // p_{k-1}
    double* __restrict__ pcur = ((k & 1) ? a.p1 : a.p0) + off;          // p_k
    double* __restrict__ x = a.x + off;
    // split modes: the gathered operand, the vector dotted with the product at each
    // row (read with the row's staged data), and the product's destination
    const double* __restrict__ opnd =
        MODE == kSpmvBsV ? a.p0 + off : (MODE == kSpmvBsT ? a.p1 + off : pcur);   // p, s (BiCGStab)
    const double* __restrict__ partner = MODE == kSpmvBsV ? a.b + off : opnd;     // rh = b, or the operand
    double* __restrict__ out = (MODE == kSpmvBsT ? a.z : a.q) + off;              // q or v, t (BiCGStab)

    // SparseTensorList: an item that stopped in an earlier launch skips the prefetch of
    // its first tile (late launches run while most items have stopped).  A stop word
    // below k is final, so every thread reads the same decision.
    if constexpr (MODE == kSpmvFused || MODE == kSpmvSplit)
        if (a.list_wg && a.st[sys].stop_iter < k) return;
    int64_t t = tr.first;
    int64_t k0 = 0, k1 = 0, k0n = 0, k1n = 0;
    // Two stage buffers used alternately (the loop is unrolled by two), so the
    // registers of a staged tile are never copied from one buffer to the other.
    TileStage<RP, U> SA, SB;
    if (t < ntiles) {
        k0 = tile_k0(t);
        k1 = tile_k1(t);
        stage_tile<RP, CAP, OFF32, SPLIT, C16>(SA, rp, col, col16, vals, SPLIT ? partner : rin, pprev, x, tile_of(t), n, k0,
                                          k1);
    }
    if (t + Gs < ntiles) {
        k0n = tile_k0(t + Gs);
        k1n = tile_k1(t + Gs);
    }

    double beta = 0.0, alpha_prev = 0.0;
    if constexpr (MODE == kSpmvSplit) {
        // k_cg_pupd of this step wrote stop_iter = k if the system stops here
        if (tid == 0) s_stop = a.st[sys].stop_iter;
        __syncthreads();
        if (s_stop <= k) return;
    } else if constexpr (SPLIT) {
        // BiCGStab: stopped by a kernel of an earlier phase of the iteration sequence
        if (tid == 0) s_stop = a.st[sys].stop_iter;
        __syncthreads();
        if (s_stop < bs_phase(k, MODE == kSpmvBsV ? kPhaseV : kPhaseT)) return;
    } else {
    const int run = cg_step_begin(a, sys, lb, k, s_red, &s_stop, beta, alpha_prev);
    if (run == kStepStopped) return;
    if (run == kStepStopNow) {
        // Stop: apply the deferred update x_k = x_{k-1} + alpha_{k-1} p_{k-1}.
        if (!first) {
            for (int64_t m = tr.first; m < tr.len; m += tr.step) {
                const int64_t i = (tr.lo + m) * kTile + tid;
                if (i < n) {
                    const double tx = alpha_prev * pprev[i];
                    x[i] = x[i] + tx;
                }
            }
        }
        return;
    }
    }

    double* __restrict__ q = a.q + off;
    // the gathered operand: p_k formed on the fly, or (SPLIT) read as formed
    using Gather = std::conditional_t<SPLIT, GatherX<OFF32>, GatherCG<OFF32>>;
    Gather g;
    if constexpr (SPLIT) g = GatherX<OFF32>{opnd};
    else g = GatherCG<OFF32>{rin, pprev, beta};
    double sig = 0.0, tt2 = 0.0;
    // Process tile t from stage `cur` while staging the next tile into `nxt`.
    auto process = [&](TileStage<RP, U>& cur, TileStage<RP, U>& nxt) {
        const int64_t tn = t + Gs;
        const int64_t row0 = tile_of(t) * kTile;
        const int nr = static_cast<int>(min(static_cast<int64_t>(kTile), n - row0));
        const int64_t i = row0 + min(tid, nr - 1);
        const int64_t cnt = k1 - k0;
        int64_t k0nn = 0, k1nn = 0;
        if (tn + Gs < ntiles) {
            k0nn = tile_k0(tn + Gs);
            k1nn = tile_k1(tn + Gs);
        }
        double s = 0.0;
        const double ri = cur.ri, ppi = cur.ppi, xi = cur.xi;
        if constexpr (CAP == kCapSkew) {
            s = tile_rowsum_pf<RP>(rp, col, vals, row0, nr, g, s_val, s_col);
            if (tn < ntiles)
                stage_tile<RP, CAP, OFF32, SPLIT, C16>(nxt, rp, col, col16, vals, SPLIT ? partner : rin, pprev, x,
                                                       tile_of(tn), n, k0n, k1n);
        } else {
            // Every staged entry register goes to LDS (slots past the tile's entries are
            // never read), on both paths; the next tile is staged unconditionally (past the
            // workgroup's last tile: a clamped copy of it, never used).
            const int32_t cbase = C16 ? static_cast<int32_t>(row0) : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = tid + u * kBlock;
                s_val[j] = cur.v[u];
                s_col[j] = cbase + cur.c[u];
            }
            const int64_t tstg = tile_of(min(tn, ntiles - 1));
            if (cnt <= CAP) {
                const int rs = static_cast<int>(static_cast<int64_t>(cur.a0) - k0);
                const int re = (tid < nr) ? static_cast<int>(static_cast<int64_t>(cur.a1) - k0) : rs;
                __syncthreads();
                // Gathers of the row's first RC entries are issued before the next tile's
                // prefetch: the vector-memory counter completes in order, so waiting for
                // them does not wait for the prefetch.  Slots past the row's end gather
                // the lane's own row (a valid address) and are masked below.
                double pv[RC];
#pragma unroll
                for (int u = 0; u < RC; ++u) {
                    const int64_t c = (rs + u < re) ? static_cast<int64_t>(s_col[rs + u]) : i;
                    pv[u] = g(c);
                }
                stage_tile<RP, CAP, OFF32, SPLIT, C16>(nxt, rp, col, col16, vals, SPLIT ? partner : rin, pprev, x, tstg, n,
                                                       k0n, k1n, tn < ntiles);
#pragma unroll
                for (int u = 0; u < RC; ++u) {
                    const bool ok = rs + u < re;
                    const double tt = s_val[ok ? rs + u : rs] * pv[u];
                    const double sn = s + tt;
                    s = ok ? sn : s;
                }
#pragma unroll 1
                for (int j0 = rs + RC; j0 < re; j0 += RC) {   // rows longer than RC entries
                    double pw[RC];
#pragma unroll
                    for (int u = 0; u < RC; ++u) {
                        const int j = (j0 + u < re) ? j0 + u : j0;
                        pw[u] = g(s_col[j]);
                    }
#pragma unroll
                    for (int u = 0; u < RC; ++u) {
                        const bool ok = j0 + u < re;
                        const int j = ok ? j0 + u : j0;
                        const double tt = s_val[j] * pw[u];
                        const double sn = s + tt;
                        s = ok ? sn : s;
                    }
                }
                __syncthreads();
            } else {
                __syncthreads();   // the long-row path reuses s_val and s_col
                s = tile_rowsum_long<RP, RC>(rp, col, vals, row0, nr, g, s_val, s_col);
                stage_tile<RP, CAP, OFF32, SPLIT, C16>(nxt, rp, col, col16, vals, SPLIT ? partner : rin, pprev, x, tstg, n,
                                                       k0n, k1n, tn < ntiles);
            }
        }
        if (tid < nr) {
            if constexpr (SPLIT) {
                out[i] = s;
                const double u = ri * s;          // ri holds the partner's row: p_k, rh or s
                sig = sig + u;
                if constexpr (MODE == kSpmvBsT) {
                    const double w = s * s;
                    tt2 = tt2 + w;
                }
            } else {
                const double tp = beta * ppi;
                const double pi = ri + tp;           // same expression as the gathered p_k
                pcur[i] = pi;
                q[i] = s;
                const double tx = alpha_prev * ppi;   // alpha_{-1} = 0 for k = 0
                x[i] = xi + tx;
                const double u = pi * s;
                sig = sig + u;
            }
        }
        k0 = k0n;
        k1 = k1n;
        k0n = k0nn;
        k1n = k1nn;
        t = tn;
    };
#pragma unroll 1
    while (t < ntiles) {
        process(SA, SB);
        if (t >= ntiles) break;
        process(SB, SA);
    }
    sig = block_sum(sig, s_red);
    if constexpr (MODE == kSpmvBsT) tt2 = block_sum(tt2, s_red);
    if (tid == 0) {
        const int64_t slot = parts_of(a, sys, a.G).base + lb;
        a.part_sigma[slot] = sig;
        if constexpr (MODE == kSpmvBsT) a.part_tt[slot] = tt2;
    }
}

// ----------------------------------------------------------------------------------
// Banded patterns: the CG SpMV with its gathered operand held in LDS.
//
// A pattern is banded with stride S when every stored entry (i, c) has |c - i| <= kBandHalo
// or S - kBandHalo <= |c - i| <= S: 5- and 9-point stencils on a grid whose lines hold S
// (or S - 1) unknowns.  The rows are read as lines of S rows, each cut into strips of
// kTile positions; workgroup (strip, chunk) walks its strip down a range of lines.
// The row window of line l (rows l S + pos0 + [0, w)) reads the operand only inside
// three segments, lines l - 1, l and l + 1 of the strip widened by kBandHalo on each
// side.  Those live in an LDS ring of three segments, so each value of
// p_k = r_k + beta p_{k-1} is loaded from HBM and formed once, then serves all three
// windows that read it.  The plain kernel instead re-gathers rows S apart through the
// L2, which cannot hold them when S is large.  Each row still sums its entries in
// ascending order with the same rounded products, so q and p_k are bit-identical to
// the plain kernel's.
// ----------------------------------------------------------------------------------
constexpr int kSeg = kTile + 2 * kBandHalo;   // positions per segment

// Element e (0 <= e < 2^29) of a vector: uniform base plus a 32-bit byte offset.
__device__ __forceinline__ double ld32(const double* __restrict__ base, int32_t e)
{
    return *reinterpret_cast<const double*>(reinterpret_cast<const char*>(base) + (static_cast<uint32_t>(e) << 3));
}

__device__ __forceinline__ void st32(double* __restrict__ base, int32_t e, double v)
{
    *reinterpret_cast<double*>(reinterpret_cast<char*>(base) + (static_cast<uint32_t>(e) << 3)) = v;
}

#ifndef SLA_BAND_NT
#define SLA_BAND_NT 1
#endif
// Streaming accesses of the banded SpMV (entries read once, outputs written once) carry
// the non-temporal hint.
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p)
{
#if SLA_BAND_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

__device__ __forceinline__ void st32_stream(double* __restrict__ base, int32_t e, double v)
{
    double* p = reinterpret_cast<double*>(reinterpret_cast<char*>(base) + (static_cast<uint32_t>(e) << 3));
#if SLA_BAND_NT
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// 16-byte loads and stores (a pair of doubles), with the non-temporal hint when NT.
template <bool NT>
__device__ __forceinline__ double2 ld2v(const double2* p)
{
    if constexpr (NT) {
        double2 v;
        v.x = __builtin_nontemporal_load(&p->x);
        v.y = __builtin_nontemporal_load(&p->y);
        return v;
    } else {
        return *p;
    }
}

template <bool NT>
__device__ __forceinline__ void st2v(double2* p, double2 v)
{
    if constexpr (NT) {
        __builtin_nontemporal_store(v.x, &p->x);
        __builtin_nontemporal_store(v.y, &p->y);
    } else {
        *p = v;
    }
}

// Raw loads of one segment (positions tid, and tid + kTile for tid < 2 kBandHalo).
struct SegLoad {
    double r0, pp0, r1, pp1;
};

// Every lane issues the same number of loads (the lanes past the segment's end re-read
// its last position), so the compiler's counts of loads in flight are exact.  A segment
// that is not `live` (issued only to keep those counts) has every lane read one
// position: a few cache lines instead of the segment.
__device__ __forceinline__ void seg_issue(SegLoad& L, const double* __restrict__ rin,
                                          const double* __restrict__ pprev, int32_t e0, int32_t n, bool live = true)
{
    const int32_t keep = -static_cast<int32_t>(live);   // all ones or zero: a mask, not a branch
    const int tid = threadIdx.x & keep;
    const int32_t e = min(max(e0 + tid, 0), n - 1);
    L.r0 = ld32(rin, e);
    L.pp0 = ld32(pprev, e);
    const int32_t e1 = min(max(e0 + kTile + min(tid, 2 * kBandHalo - 1), 0), n - 1);
    L.r1 = ld32(rin, e1);
    L.pp1 = ld32(pprev, e1);
}

// Form p_k on the segment and store it (positions outside [0, n) hold 0; no column
// points there).  The segment's own positions [kBandHalo, kBandHalo + kTile) also keep
// p_{k-1} in s_pp (when given), for the deferred x update of that line's rows.
//
// Every lane forms its halo value too, and stores it without a branch: a lane past the
// halo stores it to its own main position, which its next store overwrites (one lane's
// LDS stores land in program order).  A halo store behind a branch lets the compiler
// sink the two halo loads into that branch, where their wait also drains every load
// issued after them (the next windows' loads, in the pipelined kernels' prologues).
__device__ __forceinline__ void seg_commit(const SegLoad& L, double* s_seg, double* s_pp, double beta, int32_t e0,
                                           int32_t n)
{
    const int tid = threadIdx.x;
    const bool halo = tid < 2 * kBandHalo;
    const int32_t e = e0 + tid;
    const int32_t e1 = e + kTile;
    const double t1 = beta * L.pp1;
    const double v1 = L.r1 + t1;
    s_seg[halo ? tid + kTile : tid] = (e1 >= 0 && e1 < n) ? v1 : 0.0;
    const double t0 = beta * L.pp0;
    const double v0 = L.r0 + t0;
    s_seg[tid] = (e >= 0 && e < n) ? v0 : 0.0;
    if (s_pp && tid >= kBandHalo) s_pp[tid - kBandHalo] = L.pp0;
    if (s_pp && tid < kBandHalo) s_pp[tid + kTile - kBandHalo] = L.pp1;
}

// Registers of one staged window: its entries, this lane's row bounds and x, and the
// raw loads of the segment one line further down.
template <int U>
struct BandStage {
    double v[U];
    int32_t c[U];
    int32_t a0, a1;
    double xi;
    SegLoad seg;
};

// Workgroup-uniform view of the band walk of one system (all indices < 2^29 and the
// row pointers 32-bit: the band analysis admits only such patterns).
struct BandWalk {
    const int32_t* __restrict__ rp;
    const int32_t* __restrict__ col;
    const int16_t* __restrict__ col16;   // C16: c minus the first row of the entry's window
    const double* __restrict__ vals;
    const double* __restrict__ rin;     // r_k
    const double* __restrict__ pprev;   // p_{k-1}
    const double* __restrict__ x;
    int32_t n;
    int32_t nnz;    // > 0
    int32_t S;      // line stride
    int32_t pos0;   // first position of this strip within a line
    int32_t w;      // positions of the strip

    __device__ __forceinline__ int32_t base(int32_t l) const { return l * S + pos0; }
    __device__ __forceinline__ int rows(int32_t l) const   // rows of window l that exist
    {
        const int32_t m = n - base(l);
        return m <= 0 ? 0 : (m < w ? m : w);
    }
    // first / end entry of window l (uniform scalar loads)
    __device__ __forceinline__ int32_t k0(int32_t l) const { return ld_rp_uniform(rp, min(base(l), n)); }
    __device__ __forceinline__ int32_t k1(int32_t l) const { return ld_rp_uniform(rp, min(base(l) + rows(l), n)); }
};

// Issue the loads of window l (entries [k0, k1), row bounds, x) and of segment l + 1.
// C16: the columns come as 16-bit offsets from the window's first row (sign-extended
// by the load itself), which is what band_operand needs.  A window past the block's
// last line l1 is issued only to keep the load counts exact: its entry range is empty
// (one entry read) and its segment reads one position of the block's last segment.
// Its row bounds and x are still the window's (clamping those rows as well made the
// compiler reuse registers of loads in flight at the next block's start, and wait for
// all of them there).
template <int U, bool C16>
__device__ __forceinline__ void band_stage(const BandWalk& W, BandStage<U>& B, int32_t l, int32_t l1, int32_t k0,
                                           int32_t k1)
{
    const int tid = threadIdx.x;
    const bool live = l < l1;
    const int nr = W.rows(l);
    const int32_t i = min(W.base(l) + min(tid, max(nr - 1, 0)), W.n - 1);
    const int32_t* __restrict__ rpi = W.rp + i;
    B.a0 = rpi[0];
    B.a1 = rpi[1];
    B.xi = ld32(W.x, i);
    // unconditional (clamped) loads: an empty window re-reads entry min(k0, nnz - 1)
    const int32_t cnt = k1 - k0;
    const int32_t kb = cnt > 0 ? k0 : min(k0, W.nnz - 1);
    const double* __restrict__ vb = W.vals + kb;
    const int last = max(cnt - 1, 0);
    if constexpr (C16) {
        const int16_t* __restrict__ cb = W.col16 + kb;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(tid + u * kBlock, last);
            B.v[u] = ld_stream(vb + j);
            B.c[u] = ld_stream(cb + j);
        }
    } else {
        const int32_t* __restrict__ cb = W.col + kb;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(tid + u * kBlock, last);
            B.v[u] = ld_stream(vb + j);
            B.c[u] = ld_stream(cb + j);
        }
    }
    seg_issue(B.seg, W.rin, W.pprev, W.base(min(l, l1 - 1) + 1) - kBandHalo, W.n, live);
}

// LDS of one staged window besides its entries: this lane's row bounds (relative to
// the window's first entry) and x.  Kept in LDS rather than in the registers the loads
// wrote, so that summing the window never waits on the vector-memory counter while the
// next window's loads are in flight.
struct BandRows {
    int32_t rs[kTile];
    int32_t re[kTile];
    double xi[kTile];
};

// Write stage B (window l's entries [k0, k0 + cnt), segment l + 1) into LDS.
template <int U>
__device__ __forceinline__ void band_commit(const BandWalk& W, const BandStage<U>& B, int32_t l, int32_t k0,
                                            int32_t cnt, double* s_val, int32_t* s_col, BandRows* s_rows,
                                            double* s_seg, double* s_pp, double beta)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = tid + u * kBlock;
        if (j < cnt) {
            s_val[j] = B.v[u];
            s_col[j] = B.c[u];
        }
    }
    const int nr = W.rows(l);
    s_rows->rs[tid] = B.a0 - k0;
    s_rows->re[tid] = (tid < nr) ? B.a1 - k0 : B.a0 - k0;
    s_rows->xi[tid] = B.xi;
    seg_commit(B.seg, s_seg, s_pp, beta, W.base(l + 1) - kBandHalo, W.n);
}

// Operand p_k at column c for window base b, from the segment holding it (slots sp,
// so, sn hold lines l - 1, l, l + 1).  The band analysis admits a pattern only if every
// column of every window falls in one of the three segments (an entry at distance
// |d| <= kBandHalo lands in segment l, one at S - kBandHalo <= |d| <= S in segment
// l +- 1), so no column is gathered from memory.  The position is clamped into the
// segment all the same, so LDS reads stay inside the ring whatever the pattern.
__device__ __forceinline__ double band_operand(int32_t c, int32_t b, int32_t S, const double* s_p, int sp, int so,
                                               int sn)
{
    const int32_t d = c - b + kBandHalo + S;   // 0 at the first position of segment l - 1
    const int32_t o = d - S * ((d >= S) + (d >= 2 * S));
    const int slot = d >= 2 * S ? sn : (d >= S ? so : sp);
    return s_p[slot * kSeg + min(max(o, 0), kSeg - 1)];
}

// Outputs of this lane's row of one window, held until they are stored.
struct BandOut {
    int32_t i;   // row, or -1 if the lane has none
    double p, q, x;
};

// Row sum of this lane's row in window l (entries staged in LDS), and the row's
// outputs: p_k, q = (A p_k)_i and the deferred update x_k = x_{k-1} + alpha_{k-1} p_{k-1}.
template <int CAP, bool C16>
__device__ __forceinline__ BandOut band_window(const BandWalk& W, int32_t l, const double* s_val,
                                               const int32_t* s_col, const BandRows* s_rows, const double* s_p,
                                               const double* s_pp, int sp, int so, int sn, int po, double alpha_prev)
{
    constexpr int RC = row_chunk(CAP);
    const int tid = threadIdx.x;
    const int32_t base = W.base(l);
    const int nr = W.rows(l);
    const int rs = s_rows->rs[tid];
    const int re = s_rows->re[tid];
    double s = 0.0;
    for (int j0 = rs; j0 < re; j0 += RC) {
        double pv[RC];
#pragma unroll
        for (int u = 0; u < RC; ++u) {
            const int j = (j0 + u < re) ? j0 + u : j0;
            pv[u] = band_operand(s_col[j], C16 ? 0 : base, W.S, s_p, sp, so, sn);
        }
#pragma unroll
        for (int u = 0; u < RC; ++u) {
            const bool ok = j0 + u < re;
            const int j = ok ? j0 + u : j0;
            const double tt = s_val[j] * pv[u];
            const double sn2 = s + tt;
            s = ok ? sn2 : s;
        }
    }
    BandOut o;
    o.i = tid < nr ? base + tid : -1;
    o.p = s_p[so * kSeg + kBandHalo + tid];
    o.q = s;
    const double tx = alpha_prev * s_pp[po * kTile + tid];   // alpha_{-1} = 0 for k = 0
    o.x = s_rows->xi[tid] + tx;
    return o;
}

__device__ __forceinline__ void band_store(const BandOut& o, double* __restrict__ pcur, double* __restrict__ q,
                                           double* __restrict__ x, double& sig)
{
    if (o.i >= 0) {
        st32_stream(pcur, o.i, o.p);
        st32_stream(q, o.i, o.q);
        st32_stream(x, o.i, o.x);
        const double u = o.p * o.q;
        sig = sig + u;
    }
}

// LDS of the banded SpMV.
template <int CAP>
struct BandLds {
    double val[CAP];
    int32_t col[CAP];
    double p[3 * kSeg];     // p_k on lines l-1, l, l+1 (ring)
    double pp[2 * kTile];   // p_{k-1} at the rows of lines l, l+1 (ring)
    BandRows rows;
};

// One block: lines [l0, l1) of the strip W describes.  Pipeline: while window l is
// summed from LDS, the loads of windows l + 1 and l + 2 (entries, bounds, x, segments
// l + 2 and l + 3) are in flight in registers and the entry range of window l + 3 is
// being read, so no load waits on another load's result.  Every load is unconditional
// and every path that continues the loop passes a commit, so the compiler's wait counts
// are exact and a commit leaves the newer window's loads in flight.
template <int CAP, bool C16>
__device__ __forceinline__ void band_block(const BandWalk& W, int32_t l0, int32_t l1, BandLds<CAP>& L, double beta,
                                           double alpha_prev, double* __restrict__ pcur, double* __restrict__ q,
                                           double* __restrict__ x, double& sig)
{
    constexpr int U = CAP / kBlock;
    const int32_t n = W.n;
    BandStage<U> SA, SB;
    SegLoad Em, E0;   // segments of lines l0 - 1 and l0
    // entry ranges [k0, k1) of windows l, l + 1, l + 2
    int32_t k0a = W.k0(l0), k1a = W.k1(l0), k0b = 0, k1b = 0, k0c = 0, k1c = 0;
    band_stage<U, C16>(W, SA, l0, l1, k0a, k1a);
    seg_issue(Em, W.rin, W.pprev, W.base(l0 - 1) - kBandHalo, n);
    seg_issue(E0, W.rin, W.pprev, W.base(l0) - kBandHalo, n);
    if (l0 + 1 < l1) {
        k0b = W.k0(l0 + 1);
        k1b = W.k1(l0 + 1);
    }
    band_stage<U, C16>(W, SB, l0 + 1, l1, k0b, k1b);
    if (l0 + 2 < l1) {
        k0c = W.k0(l0 + 2);
        k1c = W.k1(l0 + 2);
    }
    // Ring slots: line l - 1 in sp, l in so, l + 1 in sn; p_{k-1} of line l in po.
    int sp = 0, so = 1, sn = 2, po = 0;
    seg_commit(Em, L.p + sp * kSeg, nullptr, beta, W.base(l0 - 1) - kBandHalo, n);
    seg_commit(E0, L.p + so * kSeg, L.pp + po * kTile, beta, W.base(l0) - kBandHalo, n);
    band_commit(W, SA, l0, k0a, k1a - k0a, L.val, L.col, &L.rows, L.p + sn * kSeg, L.pp + (po ^ 1) * kTile, beta);
    __syncthreads();
    int32_t l = l0;
    // One window l, with window l + 1's loads already in flight in `nb`: issue window
    // l + 2's loads into `na` (free: its window l was committed), read the range of
    // window l + 3, sum window l, commit `nb`, then store window l's rows (after the
    // commit's wait, so that wait never includes them).  Two windows per trip so the
    // stage buffers alternate in place.
#define SLA_BAND_WINDOW(na, nb)                                                                            \
    {                                                                                                      \
        int32_t k0d = 0, k1d = 0;                                                                          \
        band_stage<U, C16>(W, na, l + 2, l1, k0c, k1c); /* past l1: one row, exact counts */          \
        if (l + 3 < l1) {                                                                                  \
            k0d = W.k0(l + 3);                                                                             \
            k1d = W.k1(l + 3);                                                                             \
        }                                                                                                  \
        const BandOut o = band_window<CAP, C16>(W, l, L.val, L.col, &L.rows, L.p, L.pp, sp, so, sn, po, alpha_prev); \
        __syncthreads(); /* window l's LDS reads are done: rotate the rings */                            \
        const int t3 = sp;                                                                                 \
        sp = so;                                                                                           \
        so = sn;                                                                                           \
        sn = t3;                                                                                           \
        po ^= 1;                                                                                           \
        ++l;                                                                                               \
        k0a = k0b;                                                                                         \
        k1a = k1b;                                                                                         \
        k0b = k0c;                                                                                         \
        k1b = k1c;                                                                                         \
        k0c = k0d;                                                                                         \
        k1c = k1d;                                                                                         \
        if (l >= l1) {                                                                                     \
            band_store(o, pcur, q, x, sig);                                                                \
            break;                                                                                         \
        }                                                                                                  \
        band_commit(W, nb, l, k0a, k1a - k0a, L.val, L.col, &L.rows, L.p + sn * kSeg,                      \
                    L.pp + (po ^ 1) * kTile, beta);                                                        \
        band_store(o, pcur, q, x, sig);                                                                    \
        __syncthreads();                                                                                   \
    }
#pragma unroll 1
    while (l < l1) {
        SLA_BAND_WINDOW(SA, SB)
        SLA_BAND_WINDOW(SB, SA)
    }
#undef SLA_BAND_WINDOW
}

// Deferred x update x_k = x_{k-1} + alpha_{k-1} p_{k-1} of the rows of every block a
// workgroup of the line-walking SpMV owns (a system that stops at iteration k).
// sw: positions per strip (kTile, or 2 kTile for the two-rows-per-lane kernel).
// First block of workgroup lb in the persistent band grid (it then takes every G-th
// block).  Workgroup lb runs on XCD lb mod 8; with G a multiple of 8, the G / 8
// workgroups of one XCD take consecutive blocks of each round of G blocks, i.e.
// neighbouring strips of a line block.  Where a grid line does not start on a 128-byte
// boundary, neighbouring strips share a cache line at their edge, and this way both
// halves meet in one XCD's L2 (one fetch, one full-line write-back) instead of two.
__device__ __forceinline__ int32_t band_first_block(int32_t lb, int32_t G)
{
    return (G & 7) ? lb : (lb & 7) * (G >> 3) + (lb >> 3);
}

__device__ __forceinline__ void band_stop_x(int32_t lb, int32_t G, int32_t nblk, int32_t strips, int32_t B,
                                            int32_t lines, int32_t S, int32_t n, double alpha_prev,
                                            const double* __restrict__ pprev, double* __restrict__ x,
                                            int32_t sw = kTile)
{
    for (int32_t b = band_first_block(lb, G); b < nblk; b += G) {
        const int32_t j = b % strips;
        const int32_t l0 = (b / strips) * B;
        const int32_t l1 = min(l0 + B, lines);
        const int32_t w = min(sw, S - j * sw);
        for (int32_t m = l0; m < l1; ++m) {
            for (int32_t t = threadIdx.x; t < w; t += kBlock) {
                const int32_t i = m * S + j * sw + t;
                if (i < n) {
                    const double tx = alpha_prev * ld32(pprev, i);
                    st32(x, i, ld32(x, i) + tx);
                }
            }
        }
    }
}

// Grid: (G, batch).  The blocks (strip j, lines [c B, c B + B)) are numbered
// c * strips + j, and workgroup lb takes every G-th block from band_first_block(lb, G):
// the workgroups in flight cover consecutive blocks, so they stream one front of about
// G / strips * B lines through memory together.
template <int CAP, bool C16>
__global__ __launch_bounds__(kBlock) void k_cg_spmv_band(CgArgs a, int64_t k)
{
    __shared__ BandLds<CAP> L;
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const int sys = blockIdx.y;
    const int lb = blockIdx.x;
    const int tid = threadIdx.x;
    const bool first = (k == 0);
    const int32_t n = static_cast<int32_t>(a.n);
    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const int32_t S = static_cast<int32_t>(a.band_stride);
    const int32_t lines = static_cast<int32_t>(a.band_lines);
    const int32_t B = a.band_block;
    const int32_t strips = (S + kTile - 1) / kTile;
    const int32_t nblk = strips * ((lines + B - 1) / B);
    BandWalk W;
    W.rp = static_cast<const int32_t*>(a.row_ptr);
    W.col = a.col;
    W.col16 = a.col16;
    W.vals = a.vals + static_cast<int64_t>(sys) * a.nnz;
    W.rin = gathered_r(a, first) + off;             // r_k (r_0 = b), or z_k
    W.pprev = ((k & 1) ? a.p0 : a.p1) + off;       // p_{k-1}
    double* __restrict__ pcur = ((k & 1) ? a.p1 : a.p0) + off;   // p_k
    double* __restrict__ x = a.x + off;
    W.x = x;
    W.n = n;
    W.nnz = static_cast<int32_t>(a.nnz);
    W.S = S;

    double beta, alpha_prev;
    const int run = cg_step_begin(a, sys, lb, k, s_red, &s_stop, beta, alpha_prev);
    if (run == kStepStopped) return;
    if (run == kStepStopNow) {
        if (!first) band_stop_x(lb, a.G, nblk, strips, B, lines, S, n, alpha_prev, W.pprev, x);
        return;
    }
    double* __restrict__ q = a.q + off;
    double sig = 0.0;
#pragma unroll 1
    for (int32_t b = band_first_block(lb, a.G); b < nblk; b += a.G) {
        const int32_t j = b % strips;
        const int32_t l0 = (b / strips) * B;
        W.pos0 = j * kTile;
        W.w = min(kTile, S - W.pos0);
        band_block<CAP, C16>(W, l0, min(l0 + B, lines), L, beta, alpha_prev, pcur, q, x, sig);
        __syncthreads();   // the next block refills the LDS
    }
    sig = block_sum(sig, s_red);
    if (tid == 0) a.part_sigma[static_cast<int64_t>(sys) * a.G + lb] = sig;
}

// ----------------------------------------------------------------------------------
// Banded patterns in the diagonal layout: the line-walking CG SpMV without staging
// entries.
//
// A banded pattern whose stored offsets c - i take at most kDiaMax distinct values
// (the pattern's "diagonals") keeps one value per diagonal and row, [d][i], and per row
// a bit mask of the diagonals it stores.  The values are copied into that layout once
// per solve (k_dia_vals).  The SpMV then gives lane t the row t of each window: it reads
// that row's values, its mask and x (all coalesced across the window's lanes: no column
// indices, no row pointers, no LDS staging of entries) and takes every operand from the
// LDS ring of three line segments that k_cg_spmv_band keeps.  Diagonals are summed in
// ascending offset, which is ascending column order, and those a row does not store are
// skipped, so every row sum equals the CSR row sum to the last bit.
// ----------------------------------------------------------------------------------

// Code of offset delta = c - i in a pattern of line stride S, or -1 if it has none.
__device__ __forceinline__ int dia_code(int32_t delta, int32_t S)
{
    const int b = delta < -kBandHalo ? -1 : (delta > kBandHalo ? 1 : 0);
    const int32_t e = delta - b * S;
    if (e < -kBandHalo || e > kBandHalo) return -1;
    return (b + 1) * kDiaCodesPerBand + static_cast<int>(e) + kBandHalo;
}

__global__ __launch_bounds__(kBlock) void k_dia_codes(const int32_t* __restrict__ rp, const int32_t* __restrict__ col,
                                                      int64_t n, int32_t S, uint32_t* out)
{
    __shared__ uint32_t s_bits[3];
    if (threadIdx.x < 3) s_bits[threadIdx.x] = 0;
    __syncthreads();
    uint32_t lo = 0, hi = 0, bad = 0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kBlock) {
        for (int32_t k = rp[i]; k < rp[i + 1]; ++k) {
            const int c = dia_code(col[k] - static_cast<int32_t>(i), S);
            if (c < 0) bad = 1u;
            else if (c < 32) lo |= 1u << c;
            else hi |= 1u << (c - 32);
        }
    }
    if (lo) atomicOr(&s_bits[0], lo);
    if (hi) atomicOr(&s_bits[1], hi);
    if (bad) atomicOr(&s_bits[2], 1u);
    __syncthreads();
    if (threadIdx.x < 3 && s_bits[threadIdx.x]) atomicOr(out + threadIdx.x, s_bits[threadIdx.x]);
}

template <typename MT>
__global__ __launch_bounds__(kBlock) void k_dia_mask(const int32_t* __restrict__ rp, const int32_t* __restrict__ col,
                                                     int64_t n, int32_t S, DiaMap m, MT* __restrict__ mask)
{
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kBlock) {
        uint32_t bits = 0;
        for (int32_t k = rp[i]; k < rp[i + 1]; ++k) {
            const int c = dia_code(col[k] - static_cast<int32_t>(i), S);
            const int d = c < 0 ? -1 : m.d_of_code[c];
            if (d >= 0) bits |= 1u << d;
        }
        mask[i] = static_cast<MT>(bits);
    }
}

__global__ __launch_bounds__(kBlock) void k_dia_vals(const int32_t* __restrict__ rp, const int32_t* __restrict__ col,
                                                     const double* __restrict__ vals, int64_t n, int64_t nnz,
                                                     int32_t S, DiaMap m, int nd, double* __restrict__ out)
{
    const int sys = blockIdx.y;
    const double* __restrict__ v = vals + static_cast<int64_t>(sys) * nnz;
    double* __restrict__ o = out + static_cast<int64_t>(sys) * nd * n;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kBlock) {
        for (int32_t k = rp[i]; k < rp[i + 1]; ++k) {
            const int c = dia_code(col[k] - static_cast<int32_t>(i), S);
            const int d = c < 0 ? -1 : m.d_of_code[c];
            if (d >= 0) o[static_cast<int64_t>(d) * n + i] = v[k];
        }
    }
}

// Registers of one staged window: this lane's row values (one per diagonal slot), its
// mask and x, and the raw loads of the segment one line further down.
template <int ND>
struct DiaStage {
    double v[ND];
    uint32_t m;
    double xi;
    SegLoad seg;
};

// Segments of the diagonal-layout SpMV: kDiaSeg positions from seg0(m), kDiaMargin
// before the strip's origin (less the line's shift), so that each holds what the
// windows of lines m - 1, m and m + 1 read from line m, shifted or not.
constexpr int kDiaMargin = 16;
constexpr int kDiaSeg = kTile + 2 * kDiaMargin;

template <int ND>
struct DiaWalk {
    const double* vd[ND];               // diagonal d of this system (slots past nd repeat the last)
    const void* mask;
    const double* __restrict__ rin;     // r_k
    const double* __restrict__ pprev;   // p_{k-1}
    const double* __restrict__ x;
    int32_t n;
    int32_t S;
    int32_t nd;
    int32_t pos0;   // first position of the strip within a line (j kTile)
    int32_t j;      // the strip
    int32_t last;   // the last strip of a line
    int32_t sh;     // 8 when the windows are aligned (S = 8 mod 16), else 0
    // Line l's shift: with S = 8 (mod 16) every odd line starts 64 bytes past a 128-byte
    // boundary; its windows after the first start delta(l) rows before the strip's
    // origin, which puts them (and their values, masks, x and outputs) on one.
    __device__ __forceinline__ int32_t delta(int32_t l) const { return sh & -(l & 1); }
    __device__ __forceinline__ int32_t base(int32_t l) const { return l * S + pos0 - (j > 0 ? delta(l) : 0); }
    __device__ __forceinline__ int32_t end(int32_t l) const
    {
        return j == last ? (l + 1) * S : l * S + pos0 + kTile - delta(l);
    }
    __device__ __forceinline__ int rows(int32_t l) const   // rows of window l that exist (<= kTile)
    {
        const int32_t m = min(end(l), n) - base(l);
        return m <= 0 ? 0 : m;
    }
    __device__ __forceinline__ int32_t seg0(int32_t m) const { return m * S + pos0 - delta(m) - kDiaMargin; }
    // position of window m's first row in line m's segment (its p_{k-1} for the x update)
    __device__ __forceinline__ int32_t own0(int32_t m) const { return kDiaMargin + (j > 0 ? 0 : delta(m)); }
};

// Segment loads of the diagonal-layout SpMV: kTile positions from e0 and kDiaSeg - kTile
// more (every lane issues both; `live` as in seg_issue).
__device__ __forceinline__ void dia_seg_issue(SegLoad& L, const double* __restrict__ rin,
                                              const double* __restrict__ pprev, int32_t e0, int32_t n, bool live)
{
    const int32_t keep = -static_cast<int32_t>(live);   // all ones or zero: a mask, not a branch
    const int tid = threadIdx.x & keep;
    const int32_t e = min(max(e0 + tid, 0), n - 1);
    L.r0 = ld32(rin, e);
    L.pp0 = ld32(pprev, e);
    const int32_t e1 = min(max(e0 + kTile + min(tid, kDiaSeg - kTile - 1), 0), n - 1);
    L.r1 = ld32(rin, e1);
    L.pp1 = ld32(pprev, e1);
}

// p_k on the segment (positions outside [0, n) hold 0), and, when s_pp is given, the
// window's own p_{k-1} (positions own0 ... own0 + kTile - 1) into s_pp.  Stores without
// a branch on the halo, as seg_commit.
__device__ __forceinline__ void dia_seg_commit(const SegLoad& L, double* s_seg, double* s_pp, double beta,
                                               int32_t e0, int32_t n, int32_t own0)
{
    const int tid = threadIdx.x;
    const bool halo = tid < kDiaSeg - kTile;
    const int32_t e = e0 + tid;
    const int32_t e1 = e + kTile;
    const double t1 = beta * L.pp1;
    const double v1 = L.r1 + t1;
    s_seg[halo ? tid + kTile : tid] = (e1 >= 0 && e1 < n) ? v1 : 0.0;
    const double t0 = beta * L.pp0;
    const double v0 = L.r0 + t0;
    s_seg[tid] = (e >= 0 && e < n) ? v0 : 0.0;
    if (s_pp && tid >= own0) s_pp[tid - own0] = L.pp0;
    if (s_pp && tid < own0) s_pp[tid + kTile - own0] = L.pp1;
}

// Element e (0 <= e < 2^29) of a streamed array: uniform base plus a 32-bit byte
// offset, with the non-temporal hint.
template <typename T>
__device__ __forceinline__ T ld32_stream(const T* __restrict__ base, int32_t e)
{
    return ld_stream(reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) +
                                                (static_cast<uint32_t>(e) * static_cast<uint32_t>(sizeof(T)))));
}

// Issue the loads of window l (every load unconditional: slots past nd re-read the
// last diagonal, rows past the window re-read its last row; both are masked).  Windows
// past the block's last line l1 are issued only to keep the pipeline's load counts
// exact: every lane reads the first row of the block's last window (and one position of
// the segment below it), which the last real stage has just brought into the cache.
// The diagonals' bases are separate uniform pointers (one scalar base per load, the
// row as a 32-bit offset), which keeps 64-bit address arithmetic out of the vector
// registers the loads in flight are writing.
template <int ND, bool M16>
__device__ __forceinline__ void dia_stage(const DiaWalk<ND>& W, DiaStage<ND>& B, int32_t l, int32_t l1)
{
    const int tid = threadIdx.x;
    const bool live = l < l1;
    const int32_t ll = min(l, l1 - 1);
    const int nr = W.rows(ll) & -static_cast<int>(live);   // a mask, not a branch
    const int32_t i = min(W.base(ll) + min(tid, max(nr - 1, 0)), W.n - 1);
#pragma unroll
    for (int d = 0; d < ND; ++d) B.v[d] = ld32_stream(W.vd[d], i);
    if constexpr (M16) B.m = ld32_stream(static_cast<const uint16_t*>(W.mask), i);
    else B.m = ld32_stream(static_cast<const uint8_t*>(W.mask), i);
    B.xi = ld32(W.x, i);
    dia_seg_issue(B.seg, W.rin, W.pprev, W.seg0(ll + 1), W.n, live);
}

// LDS of one committed window of the diagonal-layout SpMV: its rows' values by
// diagonal, masks and x.  Kept in LDS rather than in the registers the loads wrote (as
// in band_block), so summing the window never waits on the vector-memory counter while
// the next windows' loads are in flight.
template <int ND>
struct DiaRows {
    double v[ND][kTile];
    double xi[kTile];
    uint32_t m[kTile];
};

template <int ND>
__device__ __forceinline__ void dia_commit(const DiaWalk<ND>& W, const DiaStage<ND>& B, int32_t l, DiaRows<ND>* R,
                                           double* s_seg, double* s_pp, double beta)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int d = 0; d < ND; ++d) R->v[d][tid] = B.v[d];
    R->xi[tid] = B.xi;
    R->m[tid] = B.m;
    dia_seg_commit(B.seg, s_seg, s_pp, beta, W.seg0(l + 1), W.n, W.own0(l + 1));
}

// One block: lines [l0, l1) of the strip W describes, pipelined as band_block: while
// window l is summed from LDS, the loads of windows l + 1 and l + 2 (values, masks, x,
// segments l + 2 and l + 3) are in flight in the two stage buffers, which alternate in
// place (the loop is unrolled by two).  A third buffer (three windows in flight) and
// two workgroups per CU both measured slower at 169M rows.
template <int ND, bool M16>
__device__ __forceinline__ void dia_block(const DiaWalk<ND>& W, const CgArgs& a, int32_t l0, int32_t l1, double* s_p,
                                          double* s_pp, DiaRows<ND>* R, double beta, double alpha_prev,
                                          double* __restrict__ pcur, double* __restrict__ q, double* __restrict__ x,
                                          double& sig)
{
    const int tid = threadIdx.x;
    const int32_t n = W.n;
    DiaStage<ND> SA, SB;
    SegLoad Em, E0;
    dia_stage<ND, M16>(W, SA, l0, l1);
    dia_seg_issue(Em, W.rin, W.pprev, W.seg0(l0 - 1), n, true);
    dia_seg_issue(E0, W.rin, W.pprev, W.seg0(l0), n, true);
    dia_stage<ND, M16>(W, SB, l0 + 1, l1);
    int sp = 0, so = 1, sn = 2, po = 0;
    dia_seg_commit(Em, s_p + sp * kDiaSeg, nullptr, beta, W.seg0(l0 - 1), n, 0);
    dia_seg_commit(E0, s_p + so * kDiaSeg, s_pp + po * kTile, beta, W.seg0(l0), n, W.own0(l0));
    dia_commit<ND>(W, SA, l0, R, s_p + sn * kDiaSeg, s_pp + (po ^ 1) * kTile, beta);
    __syncthreads();
    int32_t l = l0;
    // Window l, window l + 1's loads in flight in `nb`: issue window l + 2's loads into
    // `na` (free: its window was committed), sum window l, rotate the rings, commit
    // `nb`, then store window l's outputs (after the commit's wait, so that wait never
    // includes them).
#define SLA_DIA_WINDOW(na, nb)                                                                            \
    {                                                                                                     \
        dia_stage<ND, M16>(W, na, l + 2, l1); /* past l1: one row, exact counts */                        \
        double s = 0.0;                                                                                   \
        const uint32_t msk = R->m[tid];                                                                   \
        /* where row base(l) + tid's position sits in the segments of lines l - 1, l, l + 1 */            \
        const int32_t dl = W.j > 0 ? W.delta(l) : 0;                                                      \
        const int32_t offm = kDiaMargin + W.delta(l - 1) - dl;                                            \
        const int32_t off0 = kDiaMargin + W.delta(l) - dl;                                                \
        const int32_t offp = kDiaMargin + W.delta(l + 1) - dl;                                            \
        _Pragma("unroll") for (int d = 0; d < ND; ++d)                                                    \
        {                                                                                                 \
            const int sb = a.dia_b[d];                                                                    \
            const int seg = sb < 0 ? sp : (sb > 0 ? sn : so);                                             \
            const int32_t ob = sb < 0 ? offm : (sb > 0 ? offp : off0);                                    \
            const double pv = s_p[seg * kDiaSeg + a.dia_e[d] + ob + tid];                                 \
            const double t = R->v[d][tid] * pv;                                                           \
            const double s2 = s + t;                                                                      \
            s = ((msk >> d) & 1u) ? s2 : s;                                                               \
        }                                                                                                 \
        const bool own = tid < W.rows(l);                                                                 \
        const int32_t i = W.base(l) + tid;                                                                \
        const double pk = s_p[so * kDiaSeg + off0 + tid];                                                 \
        const double tx = alpha_prev * s_pp[po * kTile + tid]; /* alpha_{-1} = 0 for k = 0 */             \
        const double xo = R->xi[tid] + tx;                                                                \
        __syncthreads(); /* window l's LDS reads are done: rotate the rings */                            \
        const int t3 = sp;                                                                                \
        sp = so;                                                                                          \
        so = sn;                                                                                          \
        sn = t3;                                                                                          \
        po ^= 1;                                                                                          \
        ++l;                                                                                              \
        if (l < l1) dia_commit<ND>(W, nb, l, R, s_p + sn * kDiaSeg, s_pp + (po ^ 1) * kTile, beta);       \
        if (own) {                                                                                        \
            st32_stream(pcur, i, pk);                                                                     \
            st32_stream(q, i, s);                                                                         \
            st32_stream(x, i, xo);                                                                        \
            const double u = pk * s;                                                                      \
            sig = sig + u;                                                                                \
        }                                                                                                 \
        if (l >= l1) break;                                                                               \
        __syncthreads();                                                                                  \
    }
#pragma unroll 1
    while (l < l1) {
        SLA_DIA_WINDOW(SA, SB)
        SLA_DIA_WINDOW(SB, SA)
    }
#undef SLA_DIA_WINDOW
}

// Grid and blocks as k_cg_spmv_band.
template <int ND, bool M16>
__global__ __launch_bounds__(kBlock) void k_cg_spmv_dia(CgArgs a, int64_t k)
{
    __shared__ double s_p[3 * kDiaSeg];
    __shared__ double s_pp[2 * kTile];
    __shared__ DiaRows<ND> s_rows;
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const int sys = blockIdx.y;
    const int lb = blockIdx.x;
    const int tid = threadIdx.x;
    const bool first = (k == 0);
    const int32_t n = static_cast<int32_t>(a.n);
    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const int32_t S = static_cast<int32_t>(a.band_stride);
    const int32_t lines = static_cast<int32_t>(a.band_lines);
    const int32_t B = a.band_block;
    const int32_t strips = (S + kTile - 1) / kTile;
    const int32_t nblk = strips * ((lines + B - 1) / B);
    DiaWalk<ND> W;
#pragma unroll
    for (int d = 0; d < ND; ++d) W.vd[d] = a.dia_v[d] + static_cast<int64_t>(sys) * a.dia_nd * a.n;
    W.mask = a.dia_mask;
    W.rin = gathered_r(a, first) + off;             // r_k (r_0 = b), or z_k
    W.pprev = ((k & 1) ? a.p0 : a.p1) + off;       // p_{k-1}
    double* __restrict__ pcur = ((k & 1) ? a.p1 : a.p0) + off;   // p_k
    double* __restrict__ x = a.x + off;
    W.x = x;
    W.n = n;
    W.S = S;
    W.nd = a.dia_nd;
    W.last = strips - 1;
    W.sh = a.dia_shift;

    double beta, alpha_prev;
    const int run = cg_step_begin(a, sys, lb, k, s_red, &s_stop, beta, alpha_prev);
    if (run == kStepStopped) return;
    if (run == kStepStopNow) {
        if (!first) band_stop_x(lb, a.G, nblk, strips, B, lines, S, n, alpha_prev, W.pprev, x);
        return;
    }
    double* __restrict__ q = a.q + off;
    double sig = 0.0;
#pragma unroll 1
    for (int32_t b = band_first_block(lb, a.G); b < nblk; b += a.G) {
        const int32_t j = b % strips;
        const int32_t l0 = (b / strips) * B;
        W.pos0 = j * kTile;
        W.j = j;
        dia_block<ND, M16>(W, a, l0, min(l0 + B, lines), s_p, s_pp, &s_rows, beta, alpha_prev, pcur, q, x, sig);
        __syncthreads();   // the next block refills the ring
    }
    (void)tid;
    sig = block_sum(sig, s_red);
    if (tid == 0) a.part_sigma[static_cast<int64_t>(sys) * a.G + lb] = sig;
}

// k_cg_pupd (split schedule): the step's decisions (cg_step_begin), then for the
// workgroup's rows p_k = r_k + beta_k p_{k-1} and the deferred x_k = x_{k-1} +
// alpha_{k-1} p_{k-1}, the same expressions the fused SpMV evaluates.  Grid (Gu, batch).
__global__ __launch_bounds__(kBlock) void k_cg_pupd(CgArgs a, int64_t k)
{
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const BlockCoord bc = block_coord(a, a.Gu);
    const int sys = bc.sys;
    const int tid = threadIdx.x;
    const TileRange tr = bc.tr;
    const bool first = (k == 0);
    const int64_t off = vec_off(a, sys);
    const int64_t n = a.n;
    const double* __restrict__ rin = gathered_r(a, first) + off;
    const double* __restrict__ pprev = ((k & 1) ? a.p0 : a.p1) + off;
    double* __restrict__ pcur = ((k & 1) ? a.p1 : a.p0) + off;
    double* __restrict__ x = a.x + off;
    double beta, alpha_prev;
    const int run = cg_step_begin(a, sys, bc.lb, k, s_red, &s_stop, beta, alpha_prev);
    if (run == kStepStopped) return;
    const bool stop = (run == kStepStopNow);
    if (stop && first) return;
#pragma unroll 1
    for (int64_t m0 = tr.first; m0 < tr.len; m0 += kStreamUnroll * tr.step) {
        double rv[kStreamUnroll], pv[kStreamUnroll], xv[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t i = min((tr.lo + m0 + u * tr.step) * kTile + tid, n - 1);
            rv[u] = rin[i];
            pv[u] = pprev[i];
            xv[u] = x[i];
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t m = m0 + u * tr.step;
            const int64_t i = (tr.lo + m) * kTile + tid;
            if (m < tr.len && i < n) {
                const double tx = alpha_prev * pv[u];   // alpha_{-1} = 0 for k = 0
                x[i] = xv[u] + tx;
                if (!stop) {
                    const double tp = beta * pv[u];
                    pcur[i] = rv[u] + tp;
                }
            }
        }
    }
}

// Loads of one trip of the update kernel: kStreamUnroll tiles t0, t0 + step, ...
// (clamped indices; masked on use).  NT: with the non-temporal hint (systems far
// larger than the caches, where nothing of q or r is reused before the next pass).
template <bool NT, bool JAC>
__device__ __forceinline__ void load_trip(const TileRange& tr, int64_t m0, int64_t n, const double* __restrict__ q,
                                          const double* __restrict__ rin, const double* __restrict__ dg, double* qv,
                                          double* rv, double* dv)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
        const int64_t i = min((tr.lo + m0 + u * tr.step) * kTile + tid, n - 1);
        if constexpr (NT) {
            qv[u] = __builtin_nontemporal_load(q + i);
            rv[u] = __builtin_nontemporal_load(rin + i);
            if constexpr (JAC) dv[u] = __builtin_nontemporal_load(dg + i);
        } else {
            qv[u] = q[i];
            rv[u] = rin[i];
            if constexpr (JAC) dv[u] = dg[i];
        }
    }
}

// k_cg_update: alpha = rho / sigma, r -= alpha q, partial r^T r.  The first trip's
// loads are issued before the stop check and the reduction of the sigma partials;
// later trips are double-buffered so each trip's loads overlap the previous one.
template <bool NT, bool JAC>
__global__ __launch_bounds__(kBlock) void k_cg_update(CgArgs a, int64_t k)
{
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const BlockCoord bc = block_coord(a, a.Gu);
    const int sys = bc.sys;
    SysState* st = a.st + sys;
    const int tid = threadIdx.x;
    const int lb = bc.lb;
    const TileRange tr = bc.tr;
    const bool lead = (lb == 0 && tid == 0);
    const int64_t off = vec_off(a, sys);
    const int64_t n = a.n;
    const double* __restrict__ rin = (k == 0 ? a.b : a.r) + off;
    const double* __restrict__ q = a.q + off;
    double* __restrict__ r = a.r + off;
    const double* __restrict__ dg = JAC ? a.dg + off : nullptr;
    double* __restrict__ z = JAC ? a.z + off : nullptr;
    const int64_t trip = kStreamUnroll * tr.step;
    double qa[kStreamUnroll], ra[kStreamUnroll], qb[kStreamUnroll], rb[kStreamUnroll];
    double da[JAC ? kStreamUnroll : 1], db[JAC ? kStreamUnroll : 1];
    if (a.list_wg && st->stop_iter < k) return;   // an item stopped earlier: no prefetch
    if (tr.first < tr.len) load_trip<NT, JAC>(tr, tr.first, n, q, rin, dg, qa, ra, da);

    if (tid == 0) s_stop = st->stop_iter;
    const double sigma = reduce_parts(a.part_sigma, parts_of(a, sys, a.G), s_red);
    if (s_stop <= k) return;
    const double rho_k = st->rho[k & 1];
    if (!(sigma > 0.0)) {
        if (lead) {
            st->stop_iter = k;
            sla_cg_info inf;
            inf.iterations = k;
            inf.res_norm = sqrt(JAC ? st->rr : rho_k);
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
    double rr = 0.0, rz = 0.0;
    auto apply = [&](int64_t m0, const double* qv, const double* rv, const double* dv) {
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t m = m0 + u * tr.step;
            const int64_t i = (tr.lo + m) * kTile + tid;
            if (m < tr.len && i < n) {
                const double tq = alpha * qv[u];
                const double rn = rv[u] - tq;
                if constexpr (NT) __builtin_nontemporal_store(rn, r + i);
                else r[i] = rn;
                const double w = rn * rn;
                rr = rr + w;
                if constexpr (JAC) {
                    const double zn = rn / dv[u];   // z = M^{-1} r
                    if constexpr (NT) __builtin_nontemporal_store(zn, z + i);
                    else z[i] = zn;
                    const double wz = rn * zn;
                    rz = rz + wz;
                }
            }
        }
    };
#pragma unroll 1
    for (int64_t m0 = tr.first; m0 < tr.len; m0 += 2 * trip) {
        if (m0 + trip < tr.len) load_trip<NT, JAC>(tr, m0 + trip, n, q, rin, dg, qb, rb, db);
        apply(m0, qa, ra, da);
        if (m0 + trip >= tr.len) break;
        if (m0 + 2 * trip < tr.len) load_trip<NT, JAC>(tr, m0 + 2 * trip, n, q, rin, dg, qa, ra, da);
        apply(m0 + trip, qb, rb, db);
    }
    rr = block_sum(rr, s_red);
    if constexpr (JAC) {
        rz = block_sum(rz, s_red);
        if (tid == 0) {
            a.part_rr[parts_of(a, sys, a.Gu).base + lb] = rr;
            a.part_rho[parts_of(a, sys, a.Gu).base + lb] = rz;
        }
    } else {
        if (tid == 0) a.part_rho[parts_of(a, sys, a.Gu).base + lb] = rr;
    }
}

// k_cg_update_wide: the same step as k_cg_update (alpha = rho / sigma, r -= alpha q,
// z = M^{-1} r with Jacobi, partial r^T r and r^T z) with 16-byte accesses: thread t of
// workgroup lb takes the row pairs lb * 256 + t, then + 256 Gu, ... (grid-stride).  At
// 169M rows it streams 4.06 GB in 667 us against 753 us for the 8-byte, tile-strided
// kernel.  Requires 16-byte aligned vectors (n even, or one system) and no list; an odd
// n leaves its last row to thread 0 of workgroup 0.
template <bool NT, bool JAC>
__global__ __launch_bounds__(kBlock) void k_cg_update_wide(CgArgs a, int64_t k)
{
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const int sys = blockIdx.y;
    SysState* st = a.st + sys;
    const int tid = threadIdx.x;
    const int lb = blockIdx.x;
    const bool lead = (lb == 0 && tid == 0);
    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const int64_t n = a.n;
    const int64_t n2 = n >> 1;
    const double* __restrict__ rin = (k == 0 ? a.b : a.r) + off;
    const double* __restrict__ q = a.q + off;
    double* __restrict__ r = a.r + off;
    const double* __restrict__ dg = JAC ? a.dg + off : nullptr;
    double* __restrict__ z = JAC ? a.z + off : nullptr;
    const double2* __restrict__ q2 = reinterpret_cast<const double2*>(q);
    const double2* __restrict__ r2 = reinterpret_cast<const double2*>(rin);
    const double2* __restrict__ d2 = reinterpret_cast<const double2*>(dg);
    double2* __restrict__ w2 = reinterpret_cast<double2*>(r);
    double2* __restrict__ z2 = reinterpret_cast<double2*>(z);
    const int64_t step = static_cast<int64_t>(kBlock) * gridDim.x;
    const int64_t last = n2 > 0 ? n2 - 1 : 0;
    int64_t i = static_cast<int64_t>(lb) * kBlock + tid;
    // the first pair's loads go out before the stop check and the sigma reduction
    double2 qa{0.0, 0.0}, ra{0.0, 0.0}, da{1.0, 1.0};
    if (n2 > 0) {
        const int64_t c = min(i, last);
        qa = ld2v<NT>(q2 + c);
        ra = ld2v<NT>(r2 + c);
        if constexpr (JAC) da = ld2v<NT>(d2 + c);
    }
    if (tid == 0) s_stop = st->stop_iter;
    const double sigma = reduce_parts(a.part_sigma, parts_of(a, sys, a.G), s_red);
    if (s_stop <= k) return;
    const double rho_k = st->rho[k & 1];
    if (!(sigma > 0.0)) {
        if (lead) {
            st->stop_iter = k;
            sla_cg_info inf;
            inf.iterations = k;
            inf.res_norm = sqrt(JAC ? st->rr : rho_k);
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
    double rr = 0.0, rz = 0.0;
    auto apply1 = [&](double qv, double rv, double dv, double& rn_out, double& zn_out) {
        const double tq = alpha * qv;
        const double rn = rv - tq;
        const double w = rn * rn;
        rr = rr + w;
        rn_out = rn;
        if constexpr (JAC) {
            const double zn = rn / dv;   // z = M^{-1} r
            const double wz = rn * zn;
            rz = rz + wz;
            zn_out = zn;
        }
    };
#pragma unroll 1
    for (; i < n2; i += step) {
        // next pair's loads in flight while this pair is applied
        double2 qn{0.0, 0.0}, rn{0.0, 0.0}, dn{1.0, 1.0};
        const int64_t c = min(i + step, last);
        qn = ld2v<NT>(q2 + c);
        rn = ld2v<NT>(r2 + c);
        if constexpr (JAC) dn = ld2v<NT>(d2 + c);
        double2 ro, zo{0.0, 0.0};
        apply1(qa.x, ra.x, da.x, ro.x, zo.x);
        apply1(qa.y, ra.y, da.y, ro.y, zo.y);
        st2v<NT>(w2 + i, ro);
        if constexpr (JAC) st2v<NT>(z2 + i, zo);
        qa = qn;
        ra = rn;
        if constexpr (JAC) da = dn;
    }
    if ((n & 1) && lead) {   // the last row of an odd n
        const int64_t t = n - 1;
        double ro = 0.0, zo = 0.0;
        apply1(q[t], rin[t], JAC ? dg[t] : 1.0, ro, zo);
        r[t] = ro;
        if constexpr (JAC) z[t] = zo;
    }
    rr = block_sum(rr, s_red);
    const int64_t slot = parts_of(a, sys, a.Gu).base + lb;
    if constexpr (JAC) {
        rz = block_sum(rz, s_red);
        if (tid == 0) {
            a.part_rr[slot] = rr;
            a.part_rho[slot] = rz;
        }
    } else {
        if (tid == 0) a.part_rho[slot] = rr;
    }
}

// ----------------------------------------------------------------------------------
// BiCGStab (van der Vorst, 1992), the pages' iterative method for nonsymmetric systems
// (paperpeel page, section 1; section 3.1 "Five backends and auto-dispatch").  x0 = 0,
// shadow residual rh = r0 = b.  Iteration k runs five kernels: the stop tests and the
// direction p = r + beta (p - omega v) (k_bs_pupd), v = A p with <rh, v>
// (k_cg_spmv<..., kSpmvBsV>), alpha and s = r - alpha v with <s, s> (k_bs_s), t = A s
// with <t, s> and <t, t> (k_cg_spmv<..., kSpmvBsT>), then omega, x and r (k_bs_update).
// Grids, partial slots and the deterministic reductions are those of the CG kernels;
// scalars and stop decisions stay in device memory.  Every elementwise step rounds
// each product before the sum, in the order written.
// ----------------------------------------------------------------------------------

// Stop system sys from the leading thread of its workgroup 0: stop word = the deciding
// kernel's phase, the info record, one less running system.
__device__ __forceinline__ void bs_stop(const CgArgs& a, int sys, int64_t phase, int64_t iters, double res,
                                        int state)
{
    SysState* st = a.st + sys;
    st->stop_iter = phase;
    sla_cg_info inf;
    inf.iterations = iters;
    inf.res_norm = res;
    inf.rhs_norm = st->rhs;
    inf.state = state;
    inf.reserved = 0;
    a.info[sys] = inf;
    atomicSub(a.n_active, 1);
}

// x = 0, r = b, p = b, and the partials of <rh, r0> = <r0, r0> = <b, b>.
__global__ __launch_bounds__(kBlock) void k_bs_init(CgArgs a)
{
    __shared__ double s_red[kBlock / 64];
    const BlockCoord bc = block_coord(a, a.Gu);
    const int sys = bc.sys;
    const int tid = threadIdx.x;
    const TileRange tr = bc.tr;
    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const int64_t n = a.n;
    const double* __restrict__ b = a.b + off;
    double* __restrict__ x = a.x + off;
    double* __restrict__ r = a.r + off;
    double* __restrict__ p = a.p0 + off;
    double bb = 0.0;
#pragma unroll 1
    for (int64_t m0 = tr.first; m0 < tr.len; m0 += kStreamUnroll * tr.step) {
        double bv[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            bv[u] = b[min((tr.lo + m0 + u * tr.step) * kTile + tid, n - 1)];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t m = m0 + u * tr.step;
            const int64_t i = (tr.lo + m) * kTile + tid;
            if (m < tr.len && i < n) {
                x[i] = 0.0;
                r[i] = bv[u];
                p[i] = bv[u];
                const double w = bv[u] * bv[u];
                bb = bb + w;
            }
        }
    }
    bb = block_sum(bb, s_red);
    if (tid == 0) {
        a.part_rho[static_cast<int64_t>(sys) * a.Gu + bc.lb] = bb;
        a.part_rr[static_cast<int64_t>(sys) * a.Gu + bc.lb] = bb;
        if (bc.lb == 0) a.st[sys].stop_iter = INT64_MAX;
        if (bc.lb == 0 && sys == 0) *a.n_active = a.batch;
    }
}

// Start of iteration k: |r_k| and rho_k = <rh, r_k> from the partials, the stop tests
// (residual, budget, then the breakdowns rho_k = 0 or omega_{k-1} = 0), and for k > 0
// the direction p_k = r_k + beta (p_{k-1} - omega_{k-1} v_{k-1}) with
// beta = (rho_k / rho_{k-1}) (alpha_{k-1} / omega_{k-1}).  p_0 = b needs no pass.
__global__ __launch_bounds__(kBlock) void k_bs_pupd(CgArgs a, int64_t k)
{
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const BlockCoord bc = block_coord(a, a.Gu);
    const int sys = bc.sys;
    const int tid = threadIdx.x;
    const TileRange tr = bc.tr;
    SysState* st = a.st + sys;
    const bool lead = (bc.lb == 0 && tid == 0);
    const bool first = (k == 0);
    const int64_t phase = bs_phase(k, kPhaseP);
    if (tid == 0) s_stop = st->stop_iter;
    const double rho_k = reduce_partials(a.part_rho + static_cast<int64_t>(sys) * a.Gu, a.Gu, s_red);
    const double rr_k = reduce_partials(a.part_rr + static_cast<int64_t>(sys) * a.Gu, a.Gu, s_red);
    if (s_stop < phase) return;
    const double res = sqrt(rr_k);
    double thr;
    if (first) {
        thr = a.rtol * res;
        if (a.atol > thr) thr = a.atol;
    } else {
        thr = st->thr;
    }
    if (lead) {
        if (first) {
            st->rhs = res;
            st->thr = thr;
        }
        if (a.hist) a.hist[static_cast<int64_t>(sys) * (a.max_iter + 1) + k] = res;
    }
    const double omega = first ? 0.0 : st->omega[(k - 1) & 1];
    int code = -1;
    if (!a.fixed && res <= thr) code = SLA_CONVERGED;
    else if (k >= a.max_iter) code = SLA_MAX_ITER;
    else if (!first && (rho_k == 0.0 || omega == 0.0)) code = SLA_BREAKDOWN;
    if (code >= 0) {
        if (lead) bs_stop(a, sys, phase, k, res, code);
        return;
    }
    if (lead) {
        st->rho[k & 1] = rho_k;
        st->rr = rr_k;
    }
    if (first) return;
    const double q1 = rho_k / st->rho[(k - 1) & 1];
    const double q2 = st->alpha[(k - 1) & 1] / omega;
    const double beta = q1 * q2;
    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const int64_t n = a.n;
    const double* __restrict__ r = a.r + off;
    const double* __restrict__ v = a.q + off;
    double* __restrict__ p = a.p0 + off;
#pragma unroll 1
    for (int64_t m0 = tr.first; m0 < tr.len; m0 += kStreamUnroll * tr.step) {
        double rv[kStreamUnroll], pv[kStreamUnroll], vv[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t i = min((tr.lo + m0 + u * tr.step) * kTile + tid, n - 1);
            rv[u] = r[i];
            pv[u] = p[i];
            vv[u] = v[i];
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t m = m0 + u * tr.step;
            const int64_t i = (tr.lo + m) * kTile + tid;
            if (m < tr.len && i < n) {
                const double tv = omega * vv[u];
                const double d = pv[u] - tv;
                const double tb = beta * d;
                p[i] = rv[u] + tb;
            }
        }
    }
}

// alpha_k = rho_k / <rh, v> (zero: BREAKDOWN, NaN: NAN), s = r - alpha v, partial <s, s>.
__global__ __launch_bounds__(kBlock) void k_bs_s(CgArgs a, int64_t k)
{
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const BlockCoord bc = block_coord(a, a.Gu);
    const int sys = bc.sys;
    const int tid = threadIdx.x;
    const TileRange tr = bc.tr;
    SysState* st = a.st + sys;
    const bool lead = (bc.lb == 0 && tid == 0);
    const int64_t phase = bs_phase(k, kPhaseS);
    if (tid == 0) s_stop = st->stop_iter;
    const double d = reduce_partials(a.part_sigma + static_cast<int64_t>(sys) * a.G, a.G, s_red);
    if (s_stop < phase) return;
    if (d != d || d == 0.0) {
        if (lead) bs_stop(a, sys, phase, k, sqrt(st->rr), d != d ? SLA_NAN : SLA_BREAKDOWN);
        return;
    }
    const double alpha = st->rho[k & 1] / d;
    if (lead) st->alpha[k & 1] = alpha;
    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const int64_t n = a.n;
    const double* __restrict__ r = a.r + off;
    const double* __restrict__ v = a.q + off;
    double* __restrict__ sv = a.p1 + off;
    double ss = 0.0;
#pragma unroll 1
    for (int64_t m0 = tr.first; m0 < tr.len; m0 += kStreamUnroll * tr.step) {
        double rv[kStreamUnroll], vv[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t i = min((tr.lo + m0 + u * tr.step) * kTile + tid, n - 1);
            rv[u] = r[i];
            vv[u] = v[i];
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t m = m0 + u * tr.step;
            const int64_t i = (tr.lo + m) * kTile + tid;
            if (m < tr.len && i < n) {
                const double tv = alpha * vv[u];
                const double si = rv[u] - tv;
                sv[i] = si;
                const double w = si * si;
                ss = ss + w;
            }
        }
    }
    ss = block_sum(ss, s_red);
    if (tid == 0) a.part_aux[static_cast<int64_t>(sys) * a.Gu + bc.lb] = ss;
}

// End of iteration k.  |s| <= threshold: x += alpha p and stop (converged half-way,
// k + 1 iterations).  Otherwise omega = <t, s> / <t, t> (NaN: NAN, <t, t> = 0:
// BREAKDOWN), x = (x + alpha p) + omega s, r = s - omega t, partials <rh, r>, <r, r>.
__global__ __launch_bounds__(kBlock) void k_bs_update(CgArgs a, int64_t k)
{
    __shared__ double s_red[kBlock / 64];
    __shared__ int64_t s_stop;
    const BlockCoord bc = block_coord(a, a.Gu);
    const int sys = bc.sys;
    const int tid = threadIdx.x;
    const TileRange tr = bc.tr;
    SysState* st = a.st + sys;
    const bool lead = (bc.lb == 0 && tid == 0);
    const int64_t phase = bs_phase(k, kPhaseU);
    if (tid == 0) s_stop = st->stop_iter;
    const double ts = reduce_partials(a.part_sigma + static_cast<int64_t>(sys) * a.G, a.G, s_red);
    const double tt = reduce_partials(a.part_tt + static_cast<int64_t>(sys) * a.G, a.G, s_red);
    const double ss = reduce_partials(a.part_aux + static_cast<int64_t>(sys) * a.Gu, a.Gu, s_red);
    if (s_stop < phase) return;
    const double alpha = st->alpha[k & 1];
    const int64_t off = static_cast<int64_t>(sys) * a.n;
    const int64_t n = a.n;
    const double* __restrict__ p = a.p0 + off;
    const double* __restrict__ sv = a.p1 + off;
    const double* __restrict__ t = a.z + off;
    const double* __restrict__ rh = a.b + off;
    double* __restrict__ x = a.x + off;
    double* __restrict__ r = a.r + off;
    const double sres = sqrt(ss);
    if (!a.fixed && sres <= st->thr) {
        for (int64_t m = tr.first; m < tr.len; m += tr.step) {
            const int64_t i = (tr.lo + m) * kTile + tid;
            if (i < n) {
                const double tp = alpha * p[i];
                x[i] = x[i] + tp;
            }
        }
        if (lead) {
            if (a.hist) a.hist[static_cast<int64_t>(sys) * (a.max_iter + 1) + k + 1] = sres;
            bs_stop(a, sys, phase, k + 1, sres, SLA_CONVERGED);
        }
        return;
    }
    if (tt != tt || ts != ts || tt == 0.0) {
        if (lead) bs_stop(a, sys, phase, k, sqrt(st->rr), tt == 0.0 ? SLA_BREAKDOWN : SLA_NAN);
        return;
    }
    const double omega = ts / tt;
    if (lead) st->omega[k & 1] = omega;
    double rho1 = 0.0, rr1 = 0.0;
#pragma unroll 1
    for (int64_t m0 = tr.first; m0 < tr.len; m0 += kStreamUnroll * tr.step) {
        double xv[kStreamUnroll], pv[kStreamUnroll], svv[kStreamUnroll], tv[kStreamUnroll], hv[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t i = min((tr.lo + m0 + u * tr.step) * kTile + tid, n - 1);
            xv[u] = x[i];
            pv[u] = p[i];
            svv[u] = sv[i];
            tv[u] = t[i];
            hv[u] = rh[i];
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t m = m0 + u * tr.step;
            const int64_t i = (tr.lo + m) * kTile + tid;
            if (m < tr.len && i < n) {
                const double tp = alpha * pv[u];
                const double x1 = xv[u] + tp;
                const double tsv = omega * svv[u];
                x[i] = x1 + tsv;
                const double ttv = omega * tv[u];
                const double rn = svv[u] - ttv;
                r[i] = rn;
                const double w1 = hv[u] * rn;
                rho1 = rho1 + w1;
                const double w2 = rn * rn;
                rr1 = rr1 + w2;
            }
        }
    }
    rho1 = block_sum(rho1, s_red);
    rr1 = block_sum(rr1, s_red);
    if (tid == 0) {
        a.part_rho[static_cast<int64_t>(sys) * a.Gu + bc.lb] = rho1;
        a.part_rr[static_cast<int64_t>(sys) * a.Gu + bc.lb] = rr1;
    }
}

// ----------------------------------------------------------------------------------
// Lanczos eigensolver (the pages' .eigsh: paperpeel page, section 4.3, note to Table 5)
// with full reorthogonalization.  Step j: w = A v_j with <v_j, w> (the SpMV kernel in
// its t = A s mode), the three-term step w -= alpha_j v_j + beta_{j-1} v_{j-1}, twice
// the classical Gram-Schmidt pass w -= V (V^T w) over v_0 .. v_j (dots, their
// deterministic reduction, the update), then beta_j = |w| and v_{j+1} = w / beta_j.
// The eigenpairs of the small tridiagonal matrix are taken on the host; the Ritz
// vectors u_r = sum_l S[r][l] v_l are formed here.  All vectors are rows of V, each
// contiguous, so every pass is a coalesced stream.
// ----------------------------------------------------------------------------------

// Value at a workgroup-uniform address, read as a scalar load (read-only data).
__device__ __forceinline__ double ld_uniform(const double* p, int64_t i)
{
    typedef const __attribute__((address_space(4))) double* cptr;
    return ((cptr)(p))[i];
}

__device__ __forceinline__ int32_t ld_uniform_i(const int32_t* p, int64_t i)
{
    typedef const __attribute__((address_space(4))) int32_t* cptr;
    return ((cptr)(p))[i];
}

// Rows of this workgroup's grid-stride walk: i = blockIdx.x * kBlock + tid + t * stride.
#define LZ_ROWS(i, n)                                                                          \
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < (n);       \
         i += static_cast<int64_t>(gridDim.x) * kBlock)

__global__ __launch_bounds__(kBlock) void k_lz_norm(LzArgs a)
{
    __shared__ double s_red[kBlock / 64];
    double acc = 0.0;
    LZ_ROWS(i, a.n) {
        const double v = a.v0[i];
        const double t = v * v;
        acc = acc + t;
    }
    acc = block_sum(acc, s_red);
    if (threadIdx.x == 0) a.part[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kBlock) void k_lz_start(LzArgs a, double nrm)
{
    LZ_ROWS(i, a.n) a.V[i] = a.v0[i] / nrm;
}

// alpha_j = sum of the SpMV partials; w = (w - alpha_j v_j) - beta_{j-1} v_{j-1}.
__global__ __launch_bounds__(kBlock) void k_lz_three(LzArgs a, int64_t j)
{
    __shared__ double s_red[kBlock / 64];
    const double alpha = reduce_partials(a.part_sigma, a.G, s_red);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.alpha[j] = alpha;
    const double beta = j > 0 ? a.beta[j - 1] : 0.0;
    const double* __restrict__ vj = a.V + j * a.n;
    const double* __restrict__ vp = a.V + (j > 0 ? j - 1 : 0) * a.n;
    double* __restrict__ w = a.w;
    LZ_ROWS(i, a.n) {
        const double t1 = alpha * vj[i];
        double wi = w[i] - t1;
        if (j > 0) {
            const double t2 = beta * vp[i];
            wi = wi - t2;
        }
        w[i] = wi;
    }
}

// Partial dots <v_c, w> for c < ncols over this workgroup's kLzRows rows: w's slice is
// staged in LDS once; wave q takes the columns c = q, q + 4, ... and reduces each with
// shuffles, so no workgroup barrier is paid per column.
__global__ __launch_bounds__(kBlock) void k_lz_dots(LzArgs a, int64_t ncols)
{
    __shared__ double s_w[kLzRows];
    const int tid = threadIdx.x;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kLzRows;
    const int nr = static_cast<int>(min(static_cast<int64_t>(kLzRows), a.n - r0));
    for (int t = tid; t < nr; t += kBlock) s_w[t] = a.w[r0 + t];
    __syncthreads();
    const int lane = tid & 63, q = tid >> 6;
    constexpr int kW = kBlock / 64;
    // four columns per trip (c, c + 4, c + 8, c + 12): four independent load streams
    constexpr int kC = 4;
    for (int64_t c = q; c < ncols; c += kC * kW) {
        const double* __restrict__ v[kC];
#pragma unroll
        for (int u = 0; u < kC; ++u) {
            const int64_t cu = c + u * kW;
            v[u] = a.V + (cu < ncols ? cu : c) * a.n + r0;
        }
        double acc[kC] = {};
#pragma unroll 2
        for (int t = lane; t < nr; t += 64) {
            const double wt = s_w[t];
#pragma unroll
            for (int u = 0; u < kC; ++u) {
                const double p = v[u][t] * wt;
                acc[u] = acc[u] + p;
            }
        }
#pragma unroll
        for (int u = 0; u < kC; ++u) {
            const double sum = wave_sum(acc[u]);
            const int64_t cu = c + u * kW;
            if (lane == 0 && cu < ncols) a.part_h[cu * a.Gd + blockIdx.x] = sum;
        }
    }
}

// h[c] = sum over the Gd partials of column c, in a fixed order.
__global__ __launch_bounds__(kBlock) void k_lz_reduce(LzArgs a, int64_t ncols)
{
    __shared__ double s_red[kBlock / 64];
    for (int64_t c = blockIdx.x; c < ncols; c += gridDim.x) {
        const double v = reduce_partials(a.part_h + c * a.Gd, a.Gd, s_red);
        if (threadIdx.x == 0) a.h[c] = v;
    }
}

// w -= sum_c h[c] v_c (c ascending); with last, the partials of |w|^2.
__global__ __launch_bounds__(kBlock) void k_lz_axpy(LzArgs a, int64_t ncols, int last)
{
    __shared__ double s_red[kBlock / 64];
    double nrm = 0.0;
    constexpr int kU = 16;   // loads issued together; the sum stays in ascending c
    LZ_ROWS(i, a.n) {
        double acc = 0.0;
        const double* __restrict__ vc = a.V + i;
        int64_t c = 0;
        for (; c + kU <= ncols; c += kU) {
            double v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) v[u] = vc[(c + u) * a.n];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const double p = ld_uniform(a.h, c + u) * v[u];
                acc = acc + p;
            }
        }
        for (; c < ncols; ++c) {
            const double p = ld_uniform(a.h, c) * vc[c * a.n];
            acc = acc + p;
        }
        const double wi = a.w[i] - acc;
        a.w[i] = wi;
        const double t = wi * wi;
        nrm = nrm + t;
    }
    if (last) {
        nrm = block_sum(nrm, s_red);
        if (threadIdx.x == 0) a.part[blockIdx.x] = nrm;
    }
}

// The first pass's update and the second pass's dots in one read of V, for bases of at
// most MAXC columns: each thread keeps its row's v_0 .. v_{ncols-1} in registers, forms
// w_i -= sum_c h[c] v_c[i] (c ascending, as k_lz_axpy) and accumulates v_c[i] w_i over
// its rows of this workgroup's kLzRows; the per-column sums (waves, then the four waves
// in order) are the partials part_h[c][blockIdx.x] that k_lz_reduce sums, as after
// k_lz_dots.
template <int MAXC>
__global__ __launch_bounds__(kBlock) void k_lz_axpy_dots(LzArgs a, int ncols)
{
    __shared__ double s_w[kBlock / 64][MAXC];
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kLzRows;
    double d[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) d[c] = 0.0;
#pragma unroll 1
    for (int t = 0; t < kLzRows / kBlock; ++t) {
        const int64_t i = r0 + threadIdx.x + t * kBlock;
        if (i < a.n) {
            double v[MAXC];
#pragma unroll
            for (int c = 0; c < MAXC; ++c) v[c] = c < ncols ? a.V[static_cast<int64_t>(c) * a.n + i] : 0.0;
            double acc = 0.0;
#pragma unroll
            for (int c = 0; c < MAXC; ++c) {
                if (c < ncols) {
                    const double p = ld_uniform(a.h, c) * v[c];
                    acc = acc + p;
                }
            }
            const double wi = a.w[i] - acc;
            a.w[i] = wi;
#pragma unroll
            for (int c = 0; c < MAXC; ++c) {
                const double p = v[c] * wi;
                d[c] = d[c] + p;
            }
        }
    }
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const double sum = wave_sum(d[c]);
        if (lane == 0) s_w[wv][c] = sum;
    }
    __syncthreads();
    if (threadIdx.x < ncols) {
        const int c = threadIdx.x;
        const double tsum = (s_w[0][c] + s_w[1][c]) + (s_w[2][c] + s_w[3][c]);
        a.part_h[static_cast<int64_t>(c) * a.Gd + blockIdx.x] = tsum;
    }
}

// beta_j = |w|, v_{j+1} = w / beta_j (0 when beta_j = 0: the Krylov space is invariant).
__global__ __launch_bounds__(kBlock) void k_lz_next(LzArgs a, int64_t j)
{
    __shared__ double s_red[kBlock / 64];
    const double beta = sqrt(reduce_partials(a.part, a.Gu, s_red));
    if (blockIdx.x == 0 && threadIdx.x == 0) a.beta[j] = beta;
    double* __restrict__ vn = a.V + (j + 1) * a.n;
    LZ_ROWS(i, a.n) vn[i] = beta > 0.0 ? a.w[i] / beta : 0.0;
}

// u_r = sum_l S[r][l] v_l (l ascending) for r < k, with partials of <u_r, u_r> and
// <u_r, v0> (the caller's start vector).  KK >= k accumulators in registers (rows r >= k compute nothing used).
template <int KK>
__global__ __launch_bounds__(kBlock) void k_lz_ritz(LzArgs a)
{
    __shared__ double s_red[kBlock / 64];
    double uu[KK], uv[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) uu[r] = uv[r] = 0.0;
    LZ_ROWS(i, a.n) {
        double acc[KK];
#pragma unroll
        for (int r = 0; r < KK; ++r) acc[r] = 0.0;
        for (int64_t l = 0; l < a.m; ++l) {
            const double v = a.V[l * a.n + i];
#pragma unroll
            for (int r = 0; r < KK; ++r) {
                const double p = ld_uniform(a.S, static_cast<int64_t>(r < a.k ? r : 0) * a.m + l) * v;
                acc[r] = acc[r] + p;
            }
        }
        const double v0 = a.v0[i];
#pragma unroll
        for (int r = 0; r < KK; ++r) {
            if (r < a.k) a.U[static_cast<int64_t>(r) * a.n + i] = acc[r];
            const double t1 = acc[r] * acc[r];
            uu[r] = uu[r] + t1;
            const double t2 = acc[r] * v0;
            uv[r] = uv[r] + t2;
        }
    }
#pragma unroll
    for (int r = 0; r < KK; ++r) {
        const double su = block_sum(uu[r], s_red);
        const double sv = block_sum(uv[r], s_red);
        if (threadIdx.x == 0 && r < a.k) {
            a.part_ritz[static_cast<int64_t>(2 * r) * a.Gu + blockIdx.x] = su;
            a.part_ritz[static_cast<int64_t>(2 * r + 1) * a.Gu + blockIdx.x] = sv;
        }
    }
}

// Thick restart of the basis in place: V[r][i] = sum_{l < m} S[r][l] V[l][i] (l
// ascending) for r < lk, then V[lk][i] = V[m][i] (the next Lanczos vector).  Each
// workgroup owns a slice of `rows` consecutive i; it stages that slice of V[0..m) in LDS
// ([m][rows], m * rows <= kLzStage doubles) before any row is overwritten, so the
// product needs no second basis.
__global__ __launch_bounds__(kBlock) void k_lz_restart(LzArgs a, int64_t m, int64_t lk, int rows)
{
    extern __shared__ double s_v[];
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * rows;
    const int nr = static_cast<int>(min(static_cast<int64_t>(rows), a.n - i0));
    const int64_t staged = m * rows;
    for (int64_t t = threadIdx.x; t < staged; t += kBlock) {
        const int64_t l = t / rows;
        const int c = static_cast<int>(t - l * rows);
        s_v[t] = c < nr ? a.V[l * a.n + i0 + c] : 0.0;
    }
    __syncthreads();
    if (rows == 64) {   // one output row per wave and trip: S[r][.] is wave-uniform
        const int lane = threadIdx.x & 63;
        for (int64_t r0 = threadIdx.x >> 6; r0 < lk; r0 += kBlock / 64) {
            const int64_t r = __builtin_amdgcn_readfirstlane(static_cast<int>(r0));
            double acc = 0.0;
            for (int64_t l = 0; l < m; ++l) {
                const double p = ld_uniform(a.S, r * m + l) * s_v[l * 64 + lane];
                acc = acc + p;
            }
            if (lane < nr) a.V[r * a.n + i0 + lane] = acc;
        }
    } else {
        const int64_t outs = lk * rows;
        for (int64_t t = threadIdx.x; t < outs; t += kBlock) {
            const int64_t r = t / rows;
            const int c = static_cast<int>(t - r * rows);
            if (c >= nr) continue;
            const double* __restrict__ sr = a.S + r * m;
            double acc = 0.0;
            for (int64_t l = 0; l < m; ++l) {
                const double p = sr[l] * s_v[l * rows + c];
                acc = acc + p;
            }
            a.V[r * a.n + i0 + c] = acc;
        }
    }
    for (int c = threadIdx.x; c < nr; c += kBlock) a.V[lk * a.n + i0 + c] = a.V[m * a.n + i0 + c];
}

// u_r /= scale[r] (the signed norm: normalization and sign in one rounding).
__global__ __launch_bounds__(kBlock) void k_lz_scale(LzArgs a)
{
    LZ_ROWS(i, a.n) {
        for (int r = 0; r < a.k; ++r) {
            double* u = a.U + static_cast<int64_t>(r) * a.n + i;
            *u = *u / ld_uniform(a.scale, r);
        }
    }
}
// ------------------------------------------------------------------ block kernels (LOBPCG)
// Blocks are sets of column vectors of length n, each contiguous, named by index lists
// into a base array (column c at base + c n); the lists and the small coefficient
// matrices live on the device and are read as scalar loads.

// out[c] = A in[c] for c < q: every row's entries are read once per CH columns; each
// sum runs over the row's entries in ascending order, products rounded.
template <typename RP, int CH>
__global__ __launch_bounds__(kBlock) void k_blk_spmm(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                                     const double* __restrict__ vals, const double* __restrict__ in,
                                                     const int32_t* __restrict__ idx_in, double* __restrict__ out,
                                                     const int32_t* __restrict__ idx_out, int q, int64_t n)
{
    LZ_ROWS(i, n) {
        const int64_t e0 = ld_rp(rp, i), e1 = ld_rp(rp, i + 1);
        for (int c0 = 0; c0 < q; c0 += CH) {
            const double* __restrict__ x[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                const int c = c0 + u < q ? c0 + u : c0;
                x[u] = in + static_cast<int64_t>(ld_uniform_i(idx_in, c)) * n;
            }
            double acc[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) acc[u] = 0.0;
            for (int64_t e = e0; e < e1; ++e) {
                const double v = vals[e];
                const int32_t j = col[e];
#pragma unroll
                for (int u = 0; u < CH; ++u) {
                    const double p = v * x[u][j];
                    acc[u] = acc[u] + p;
                }
            }
#pragma unroll
            for (int u = 0; u < CH; ++u)
                if (c0 + u < q) out[static_cast<int64_t>(ld_uniform_i(idx_out, c0 + u)) * n + i] = acc[u];
        }
    }
}

// Partial Gram products part[g][a mv + b] = sum over this workgroup's row slices of
// A_a[i] B_b[i] (a < mu, b < mv).  A slice of R rows of every operand column is staged
// in LDS (R as large as 32 KiB allows, a multiple of 32, stride R + 1 against bank
// conflicts), eight loads issued before their stores.  With tpp > 1 (mu mv tpp <=
// kBlock) each pair is served by tpp threads over the rows r = sub, sub + tpp, ...,
// their sums added in order of sub at the end; otherwise pair p = tid + u kBlock keeps
// PP accumulators.
template <int PP>
__global__ __launch_bounds__(kBlock) void k_blk_gram(const double* __restrict__ A, const int32_t* __restrict__ ia,
                                                     int mu, const double* __restrict__ B,
                                                     const int32_t* __restrict__ ib, int mv, int64_t n, int R, int tpp,
                                                     double* __restrict__ part)
{
    extern __shared__ double s_g[];
    __shared__ int32_t s_idx[2 * kBlkMaxCols];
    const int tid = threadIdx.x;
    const int pad = R + 1;
    const int ncol = mu + mv;
    const int np = mu * mv;
    for (int t = tid; t < ncol; t += kBlock) s_idx[t] = t < mu ? ia[t] : ib[t - mu];
    const int sub = tid % tpp;
    const int lanes = kBlock / tpp;   // pairs served at once
    double acc[PP];
    int pa[PP], pb[PP];
#pragma unroll
    for (int u = 0; u < PP; ++u) {
        acc[u] = 0.0;
        const int p = min(tid / tpp + u * lanes, np - 1);
        pa[u] = p / mv;
        pb[u] = p - pa[u] * mv;
    }
    __syncthreads();
    const int64_t nslices = (n + R - 1) / R;
    const int total = ncol * R;
    for (int64_t sl = blockIdx.x; sl < nslices; sl += gridDim.x) {
        const int64_t r0 = sl * R;
        const int nr = static_cast<int>(min(static_cast<int64_t>(R), n - r0));
        for (int t0 = tid; t0 < total; t0 += 8 * kBlock) {
            double v[8];
            int dst[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u * kBlock;
                const bool ok = t < total;
                const int c = ok ? t / R : 0;
                const int r = t - c * R;
                const double* __restrict__ base = c < mu ? A : B;
                v[u] = (ok && r < nr) ? base[static_cast<int64_t>(s_idx[c]) * n + r0 + r] : 0.0;
                dst[u] = ok ? c * pad + r : -1;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (dst[u] >= 0) s_g[dst[u]] = v[u];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PP; ++u) {
            const double* __restrict__ xa = s_g + pa[u] * pad;
            const double* __restrict__ xb = s_g + (mu + pb[u]) * pad;
            double t = acc[u];
            for (int r = sub; r < nr; r += tpp) {
                const double p = xa[r] * xb[r];
                t = t + p;
            }
            acc[u] = t;
        }
        __syncthreads();
    }
    if (tpp > 1) {   // PP == 1: the tpp partial sums of each pair, added in order of sub
        s_g[tid] = acc[0];
        __syncthreads();
        const int p = tid / tpp;
        if (sub == 0 && p < np) {
            double t = 0.0;
            for (int j = 0; j < tpp; ++j) t = t + s_g[tid + j];
            part[static_cast<int64_t>(blockIdx.x) * np + p] = t;
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < PP; ++u) {
        const int p = tid + u * kBlock;
        if (p < np) part[static_cast<int64_t>(blockIdx.x) * np + p] = acc[u];
    }
}

// The same Gram partials for many pairs (mu mv > kBlock), in 4 x 4 register tiles: tile
// (ta, tb) holds the pairs a = 4 ta + da, b = 4 tb + db; per row a thread reads 8
// staged values for 16 products (two reads per product without tiles, which made the
// wide Rayleigh-Ritz Gram LDS-bound).  tpp threads share a tile over rows r = sub,
// sub + tpp, ..., their sums added in order of sub at the end; with PT tiles per
// thread.  Operand columns past mu (mv) read column mu - 1 (mv - 1) and are not written.
template <int PT>
__global__ __launch_bounds__(kBlock) void k_blk_gram_tiled(const double* __restrict__ A,
                                                           const int32_t* __restrict__ ia, int mu,
                                                           const double* __restrict__ B,
                                                           const int32_t* __restrict__ ib, int mv, int64_t n, int R,
                                                           int tpp, double* __restrict__ part)
{
    extern __shared__ double s_g[];
    __shared__ int32_t s_idx[2 * kBlkMaxCols];
    const int tid = threadIdx.x;
    const int pad = R + 1;
    const int ncol = mu + mv;
    const int np = mu * mv;
    const int tu = (mu + 3) / 4, tv = (mv + 3) / 4, ntile = tu * tv;
    for (int t = tid; t < ncol; t += kBlock) s_idx[t] = t < mu ? ia[t] : ib[t - mu];
    const int sub = tid % tpp;
    const int lanes = kBlock / tpp;
    double acc[PT][16];
    int ra[PT][4], rb[PT][4];
#pragma unroll
    for (int u = 0; u < PT; ++u) {
        const int tile = min(tid / tpp + u * lanes, ntile - 1);
        const int ta = tile / tv, tb = tile - ta * tv;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            ra[u][d] = min(4 * ta + d, mu - 1) * pad;
            rb[u][d] = (mu + min(4 * tb + d, mv - 1)) * pad;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[u][e] = 0.0;
    }
    __syncthreads();
    const int64_t nslices = (n + R - 1) / R;
    const int total = ncol * R;
    for (int64_t sl = blockIdx.x; sl < nslices; sl += gridDim.x) {
        const int64_t r0 = sl * R;
        const int nr = static_cast<int>(min(static_cast<int64_t>(R), n - r0));
        for (int t0 = tid; t0 < total; t0 += 8 * kBlock) {
            double v[8];
            int dst[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u * kBlock;
                const bool ok = t < total;
                const int c = ok ? t / R : 0;
                const int r = t - c * R;
                const double* __restrict__ base = c < mu ? A : B;
                v[u] = (ok && r < nr) ? base[static_cast<int64_t>(s_idx[c]) * n + r0 + r] : 0.0;
                dst[u] = ok ? c * pad + r : -1;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (dst[u] >= 0) s_g[dst[u]] = v[u];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PT; ++u) {
            for (int r = sub; r < nr; r += tpp) {
                double xa[4], xb[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    xa[d] = s_g[ra[u][d] + r];
                    xb[d] = s_g[rb[u][d] + r];
                }
#pragma unroll
                for (int da = 0; da < 4; ++da)
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        const double p = xa[da] * xb[db];
                        acc[u][da * 4 + db] = acc[u][da * 4 + db] + p;
                    }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < PT; ++u) {
        const int tile = tid / tpp + u * lanes;
        const int ta = tile / tv, tb = tile - ta * tv;
        for (int e = 0; e < 16; ++e) {
            // the tpp partial sums of this tile's entry e, added in order of sub
            s_g[tid] = acc[u][e];
            __syncthreads();
            if (sub == 0 && tile < ntile) {
                const int a = 4 * ta + e / 4, b = 4 * tb + e % 4;
                double t = 0.0;
                for (int j = 0; j < tpp; ++j) t = t + s_g[tid + j];
                if (a < mu && b < mv) part[static_cast<int64_t>(blockIdx.x) * np + a * mv + b] = t;
            }
            __syncthreads();
        }
    }
}

// Gram partials with the slice loads pipelined (n even, every column base 16-byte
// aligned).  Slice sl holds rows [sl R, sl R + R) of the ncol operand columns (ncol = mu,
// or mu + mv when B's columns are not A's), staged in LDS at stride R + 2; R is a power
// of two with ncol R <= 4096.  Thread t owns the 16-byte pieces e = t + u kBlock (column
// e / (R / 2), row pair e % (R / 2)): it issues the loads of its workgroup's next slice
// before the products of the current one, and stores them after.  The products run in
// TA x TB register tiles over (a, b); tpt threads (a power of two) share a tile over rows
// r = sub, sub + tpt, ..., their sums combined at the end by a butterfly within the wave
// and then in wave order.  Every pair's sum runs over its rows in a fixed order.
template <int TA, int TB, int PT, int U>
__global__ __launch_bounds__(kBlock) void k_blk_gram_pipe(const double* __restrict__ A,
                                                          const int32_t* __restrict__ ia, int mu,
                                                          const double* __restrict__ B,
                                                          const int32_t* __restrict__ ib, int mv, int same, int64_t n,
                                                          int lgh, int tpt, double* __restrict__ part)
{
    extern __shared__ double s_g[];
    const int tid = threadIdx.x;
    const int R2 = 1 << lgh, R = 2 * R2, pad = R + 2;
    const int ncol = same ? mu : mu + mv;
    const int E = ncol * R2;
    const int np = mu * mv;
    const int boff = same ? 0 : mu;
    const int tu = (mu + TA - 1) / TA, tv = (mv + TB - 1) / TB, ntile = tu * tv;
    const int sub = tid % tpt;
    const int lanes = kBlock / tpt;
    // this thread's pieces: source column start (row 0) and LDS offset
    const double* src[U];
    int dst[U], off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e = min(tid + u * kBlock, E - 1);   // pieces past E repeat the last one
        const int c = e >> lgh;
        const int r2 = e & (R2 - 1);
        const double* base = c < mu ? A : B;
        const int32_t ci = c < mu ? ia[c] : ib[c - mu];
        src[u] = base + static_cast<int64_t>(ci) * n;
        off[u] = 2 * r2;
        dst[u] = tid + u * kBlock < E ? c * pad + 2 * r2 : -1;
    }
    double acc[PT][TA * TB];
    int ra[PT][TA], rb[PT][TB];
#pragma unroll
    for (int p = 0; p < PT; ++p) {
        const int tile = min(tid / tpt + p * lanes, ntile - 1);
        const int ta = tile / tv, tb = tile - ta * tv;
#pragma unroll
        for (int d = 0; d < TA; ++d) ra[p][d] = min(TA * ta + d, mu - 1) * pad;
#pragma unroll
        for (int d = 0; d < TB; ++d) rb[p][d] = (boff + min(TB * tb + d, mv - 1)) * pad;
#pragma unroll
        for (int e = 0; e < TA * TB; ++e) acc[p][e] = 0.0;
    }
    const int64_t nslices = (n + R - 1) / R;
    const int64_t G = gridDim.x;
    double2 v[U];
    // the loads of slice sl (rows past n read the last pair; the store zeroes them, so
    // nothing waits on a load before the products of the slice in LDS)
    auto load = [&](int64_t sl) __attribute__((always_inline)) {
        const int64_t r0 = sl * R;
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const double2*>(src[u] + min(r0 + off[u], n - 2));
    };
    auto store = [&](int64_t sl) __attribute__((always_inline)) {
        const int64_t r0 = sl * R;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (dst[u] >= 0)
                *reinterpret_cast<double2*>(s_g + dst[u]) = r0 + off[u] < n ? v[u] : double2{0.0, 0.0};
    };
    int64_t sl = blockIdx.x;
    if (sl < nslices) {
        load(sl);
        store(sl);
    }
    __syncthreads();
    for (; sl < nslices; sl += G) {
        const int nr = static_cast<int>(min(static_cast<int64_t>(R), n - sl * R));
        // the next slice's loads (the last slice reloads itself: cache hits, never stored)
        const bool more = sl + G < nslices;
        load(more ? sl + G : sl);
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            for (int r = sub; r < nr; r += tpt) {
                double xa[TA], xb[TB];
#pragma unroll
                for (int d = 0; d < TA; ++d) xa[d] = s_g[ra[p][d] + r];
#pragma unroll
                for (int d = 0; d < TB; ++d) xb[d] = s_g[rb[p][d] + r];
#pragma unroll
                for (int da = 0; da < TA; ++da)
#pragma unroll
                    for (int db = 0; db < TB; ++db) {
                        const double q = xa[da] * xb[db];
                        acc[p][da * TB + db] = acc[p][da * TB + db] + q;
                    }
            }
        }
        __syncthreads();
        if (more) store(sl + G);
        __syncthreads();
    }
    // the tpt partial sums of each tile entry: a butterfly over the tile's lanes of one
    // wave (every lane ends with the same sum), then, for tiles wider than a wave, the
    // waves' sums added in wave order
    const int wl = min(tpt, 64);
#pragma unroll
    for (int p = 0; p < PT; ++p)
#pragma unroll
        for (int e = 0; e < TA * TB; ++e)
            for (int off = 1; off < wl; off <<= 1) acc[p][e] = acc[p][e] + __shfl_xor(acc[p][e], off, 64);
    const int wave = tid >> 6, lane = tid & 63;
    if (tpt > 64) {   // PT == 1 here (ntile <= 2)
        if (lane == 0)
#pragma unroll
            for (int e = 0; e < TA * TB; ++e) s_g[wave * TA * TB + e] = acc[0][e];
        __syncthreads();
        const int tile = tid / tpt;
        const int ta = tile / tv, tb = tile - ta * tv;
        if (sub == 0 && tile < ntile)
#pragma unroll
            for (int e = 0; e < TA * TB; ++e) {
                double t = 0.0;
                for (int w = 0; w < tpt / 64; ++w) t = t + s_g[(wave + w) * TA * TB + e];
                const int a = TA * ta + e / TB, b = TB * tb + e % TB;
                if (a < mu && b < mv) part[static_cast<int64_t>(blockIdx.x) * np + a * mv + b] = t;
            }
        return;
    }
#pragma unroll
    for (int p = 0; p < PT; ++p) {
        const int tile = tid / tpt + p * lanes;
        const int ta = tile / tv, tb = tile - ta * tv;
        if (sub == 0 && tile < ntile)
#pragma unroll
            for (int e = 0; e < TA * TB; ++e) {
                const int a = TA * ta + e / TB, b = TB * tb + e % TB;
                if (a < mu && b < mv) part[static_cast<int64_t>(blockIdx.x) * np + a * mv + b] = acc[p][e];
            }
    }
    (void)lane;
}

// Gram partials streamed like the combinations, with no staging (n even, column bases
// 16-byte aligned): NTP lanes share each pair of rows, lane t of them holding tile t, a
// TA x TB register tile of the products (columns past mu or mv repeat the last one and
// are not written).  A wave covers 64 / NTP row pairs, the grid strides over them, and
// each pair's sum runs over rows in a fixed order: a lane's rows in order, then a
// butterfly over the wave's lanes of the same tile, then the four waves in order.
template <int TA, int TB, int NTP>
__global__ __launch_bounds__(kBlock) void k_blk_gram_rt(const double* __restrict__ A, const int32_t* __restrict__ ia,
                                                        int mu, const double* __restrict__ B,
                                                        const int32_t* __restrict__ ib, int mv, int64_t n,
                                                        double* __restrict__ part)
{
    constexpr int RPW = 64 / NTP;   // row pairs of a wave
    __shared__ double s_w[kBlock / 64][NTP][TA * TB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = lane / RPW, rp = lane - t * RPW;
    const int tu = (mu + TA - 1) / TA, tv = (mv + TB - 1) / TB, ntile = tu * tv;
    const int tt = min(t, ntile - 1);
    const int ta = tt / tv, tb = tt - ta * tv;
    const double2* pa[TA];
    const double2* pb[TB];
#pragma unroll
    for (int d = 0; d < TA; ++d)
        pa[d] = reinterpret_cast<const double2*>(A + static_cast<int64_t>(ia[min(TA * ta + d, mu - 1)]) * n);
#pragma unroll
    for (int d = 0; d < TB; ++d)
        pb[d] = reinterpret_cast<const double2*>(B + static_cast<int64_t>(ib[min(TB * tb + d, mv - 1)]) * n);
    double acc[TA * TB];
#pragma unroll
    for (int e = 0; e < TA * TB; ++e) acc[e] = 0.0;
    const int64_t n2 = n >> 1;
    const int64_t step = static_cast<int64_t>(gridDim.x) * (kBlock / 64) * RPW;
    for (int64_t i2 = (static_cast<int64_t>(blockIdx.x) * (kBlock / 64) + wave) * RPW + rp; i2 < n2; i2 += step) {
        double2 xa[TA], xb[TB];
#pragma unroll
        for (int d = 0; d < TA; ++d) xa[d] = pa[d][i2];
#pragma unroll
        for (int d = 0; d < TB; ++d) xb[d] = pb[d][i2];
#pragma unroll
        for (int da = 0; da < TA; ++da)
#pragma unroll
            for (int db = 0; db < TB; ++db) {
                const double px = xa[da].x * xb[db].x;
                const double py = xa[da].y * xb[db].y;
                acc[da * TB + db] = acc[da * TB + db] + px;
                acc[da * TB + db] = acc[da * TB + db] + py;
            }
    }
#pragma unroll
    for (int e = 0; e < TA * TB; ++e)
        for (int off = 1; off < RPW; off <<= 1) acc[e] = acc[e] + __shfl_xor(acc[e], off, 64);
    if (rp == 0)
#pragma unroll
        for (int e = 0; e < TA * TB; ++e) s_w[wave][t][e] = acc[e];
    __syncthreads();
    const int np = mu * mv;
    for (int q = tid; q < NTP * TA * TB; q += kBlock) {
        const int tq = q / (TA * TB), e = q - tq * (TA * TB);
        if (tq >= ntile) continue;
        double v = 0.0;
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) v = v + s_w[w][tq][e];
        const int qa = tq / tv, qb = tq - qa * tv;
        const int a = TA * qa + e / TB, b = TB * qb + e % TB;
        if (a < mu && b < mv) part[static_cast<int64_t>(blockIdx.x) * np + a * mv + b] = v;
    }
}

// Small dense steps of LOBPCG, on the device so the host never waits for them.
constexpr int kCoefMax = SLA_EIG_MAX_K;   // widest block factored here

// Cholesky QR coefficients of a block of w <= kCoefMax columns from its Gram matrix G0
// [w][w], one wave.  scale: the columns are first taken to unit norm (G_ab / (|z_a| |z_b|)
// with |z_c| = sqrt(G_cc); a zero column fails).  G is then symmetrized and factored as
// R^T R column by column, each pivot tested against pivot times the largest diagonal
// entry; T = R^-1, times diag(1 / |z|) with scale, so that Z T has orthonormal columns.
// The sums run in the order of the textbook algorithm (ascending inner index).  flag:
// written with scale, read otherwise; a block that fails, or failed in the pass before,
// gets T = 0 (its columns become zero) and flag 0.
__global__ __launch_bounds__(64) void k_blk_orth_coef(const double* __restrict__ G0, int w, int scale, double pivot,
                                                      double* flag, double* __restrict__ T)
{
    __shared__ double s_g[kCoefMax * kCoefMax], s_l[kCoefMax * kCoefMax], s_nrm[kCoefMax];
    __shared__ double s_gmax;
    __shared__ int s_ok;
    const int t = threadIdx.x;
    const int np = w * w;
    if (t == 0) s_ok = scale ? 1 : (*flag != 0.0 ? 1 : 0);
    if (t < w) s_nrm[t] = scale ? sqrt(G0[t * w + t]) : 1.0;
    __syncthreads();
    if (t == 0)
        for (int c = 0; c < w; ++c)
            if (!(s_nrm[c] > 0.0)) s_ok = 0;
    for (int e = t; e < np; e += 64) {
        const int a = e / w, b = e - a * w;
        const double gab = scale ? G0[e] / (s_nrm[a] * s_nrm[b]) : G0[e];
        const double gba = scale ? G0[b * w + a] / (s_nrm[b] * s_nrm[a]) : G0[b * w + a];
        s_g[e] = 0.5 * (gab + gba);
        s_l[e] = 0.0;
    }
    __syncthreads();
    if (t == 0) {
        double gmax = 0.0;
        for (int a = 0; a < w; ++a) gmax = fmax(gmax, s_g[a * w + a]);
        s_gmax = gmax;
    }
    __syncthreads();
    for (int j = 0; j < w && s_ok; ++j) {   // s_ok is uniform at every test
        if (t == 0) {
            double d = s_g[j * w + j];
            for (int p = 0; p < j; ++p) d -= s_l[j * w + p] * s_l[j * w + p];
            if (d > pivot * s_gmax) s_l[j * w + j] = sqrt(d);
            else s_ok = 0;
        }
        __syncthreads();
        if (s_ok && t > j && t < w) {
            double v = s_g[t * w + j];
            for (int p = 0; p < j; ++p) v -= s_l[t * w + p] * s_l[j * w + p];
            s_l[t * w + j] = v / s_l[j * w + j];
        }
        __syncthreads();
    }
    // column c of R^-1 (R = L^T), rows c down to 0, into s_g (each lane its own column)
    if (s_ok && t < w) {
        const int c = t;
        for (int i = w - 1; i > c; --i) s_g[i * w + c] = 0.0;
        for (int i = c; i >= 0; --i) {
            double v = (i == c) ? 1.0 : 0.0;
            for (int p = i + 1; p <= c; ++p) v -= s_l[p * w + i] * s_g[p * w + c];
            s_g[i * w + c] = v / s_l[i * w + i];
        }
    }
    __syncthreads();
    const bool ok = s_ok != 0;
    for (int e = t; e < np; e += 64) T[e] = ok ? s_g[e] / s_nrm[e / w] : 0.0;
    if (t == 0) *flag = ok ? 1.0 : 0.0;
}

// tinv[i] = 1 / a_ii (binary search for column i in row i; the columns are sorted), and
// per workgroup the number of rows whose a_ii is missing, not finite or not positive
// (part[blockIdx.x], as a double).
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_blk_diag_inv(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                                         const double* __restrict__ vals, int64_t n,
                                                         double* __restrict__ tinv, double* __restrict__ part)
{
    __shared__ double s_red[kBlock / 64];
    double bad = 0.0;
    LZ_ROWS(i, n) {
        int64_t lo = ld_rp(rp, i), hi = ld_rp(rp, i + 1);
        double d = 0.0;
        bool found = false;
        while (lo < hi) {
            const int64_t mid = lo + (hi - lo) / 2;
            const int32_t c = col[mid];
            if (c == i) {
                d = vals[mid];
                found = true;
                break;
            }
            if (c < i) lo = mid + 1;
            else hi = mid;
        }
        const bool ok = found && d > 0.0 && d < HUGE_VAL;
        tinv[i] = ok ? 1.0 / d : 0.0;
        if (!ok) bad = bad + 1.0;
    }
    bad = block_sum(bad, s_red);
    if (threadIdx.x == 0) part[blockIdx.x] = bad;
}

// out[c][i] = in[c][i] * t[i] for c < q (the preconditioned residuals T R).
__global__ __launch_bounds__(kBlock) void k_blk_rowscale(const double* __restrict__ in,
                                                         const int32_t* __restrict__ idx_in,
                                                         double* __restrict__ out,
                                                         const int32_t* __restrict__ idx_out, int q, int64_t n,
                                                         const double* __restrict__ t)
{
    LZ_ROWS(i, n) {
        const double ti = t[i];
        for (int c = 0; c < q; ++c)
            out[static_cast<int64_t>(ld_uniform_i(idx_out, c)) * n + i] =
                in[static_cast<int64_t>(ld_uniform_i(idx_in, c)) * n + i] * ti;
    }
}

// out[p] = sum over g < G of part[g][p], p < np: one workgroup per p, a fixed order
// (strided partial sums, then the workgroup tree).  yproj (for a Gram C = B^T Z [b][w],
// b >= w): the projection coefficients Y [(w + b)][w] = [I; -C] instead.
__global__ __launch_bounds__(kBlock) void k_blk_reduce(const double* __restrict__ part, int G, int np,
                                                       double* __restrict__ out, double* __restrict__ yproj, int w)
{
    __shared__ double s_red[kBlock / 64];
    const int p = blockIdx.x;
    double v = 0.0;
    for (int g = threadIdx.x; g < G; g += kBlock) v = v + part[static_cast<int64_t>(g) * np + p];
    v = block_sum(v, s_red);
    if (threadIdx.x == 0) {
        if (yproj) {
            yproj[w * w + p] = -v;
            if (p < w * w) yproj[p] = (p / w == p % w) ? 1.0 : 0.0;
        } else {
            out[p] = v;
        }
    }
}

// out[c] = sum_j Y[j][c] in[j] (j ascending) for c < q (q <= QQ), Y [m][q]; with part,
// the partials part[g][c] of |out[c]|^2 over this workgroup's rows.
template <int QQ>
__global__ __launch_bounds__(kBlock) void k_blk_comb(const double* __restrict__ in, const int32_t* __restrict__ idx_in,
                                                     int m, const double* __restrict__ Y, double* __restrict__ out,
                                                     const int32_t* __restrict__ idx_out, int q, int64_t n,
                                                     double* __restrict__ part)
{
    __shared__ double s_red[kBlock / 64];
    double nrm[QQ];
#pragma unroll
    for (int u = 0; u < QQ; ++u) nrm[u] = 0.0;
    LZ_ROWS(i, n) {
        double acc[QQ];
#pragma unroll
        for (int u = 0; u < QQ; ++u) acc[u] = 0.0;
        // four inputs' loads issued together, their terms added in ascending j (eight
        // measured slower)
        int j = 0;
        for (; j + 4 <= m; j += 4) {
            double v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = in[static_cast<int64_t>(ld_uniform_i(idx_in, j + t)) * n + i];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int u = 0; u < QQ; ++u) {
                    const double p = ld_uniform(Y, static_cast<int64_t>(j + t) * q + (u < q ? u : 0)) * v[t];
                    acc[u] = acc[u] + p;
                }
            }
        }
        for (; j < m; ++j) {
            const double v = in[static_cast<int64_t>(ld_uniform_i(idx_in, j)) * n + i];
#pragma unroll
            for (int u = 0; u < QQ; ++u) {
                const double p = ld_uniform(Y, static_cast<int64_t>(j) * q + (u < q ? u : 0)) * v;
                acc[u] = acc[u] + p;
            }
        }
#pragma unroll
        for (int u = 0; u < QQ; ++u) {
            if (u < q) out[static_cast<int64_t>(ld_uniform_i(idx_out, u)) * n + i] = acc[u];
            const double t = acc[u] * acc[u];
            nrm[u] = nrm[u] + t;
        }
    }
    if (part) {
#pragma unroll
        for (int u = 0; u < QQ; ++u) {
            const double sv = block_sum(nrm[u], s_red);
            if (threadIdx.x == 0 && u < q) part[static_cast<int64_t>(blockIdx.x) * q + u] = sv;
        }
    }
}

// k_blk_comb on pairs of rows: the same sums, row by row in ascending j, with 16-byte
// loads and stores (every column base 16-byte aligned, n even), so each load moves two
// rows and a thread's four-input groups wait half as often per row.  The squared norms
// add the pair's two rows in order (a different grouping of the same terms than
// k_blk_comb's).
template <int QQ>
__global__ __launch_bounds__(kBlock) void k_blk_comb2(const double* __restrict__ in, const int32_t* __restrict__ idx_in,
                                                      int m, const double* __restrict__ Y, double* __restrict__ out,
                                                      const int32_t* __restrict__ idx_out, int q, int64_t n,
                                                      double* __restrict__ part)
{
    __shared__ double s_red[kBlock / 64];
    double nrm[QQ];
#pragma unroll
    for (int u = 0; u < QQ; ++u) nrm[u] = 0.0;
    const int64_t n2 = n >> 1;
    for (int64_t i2 = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i2 < n2;
         i2 += static_cast<int64_t>(gridDim.x) * kBlock) {
        double ax[QQ], ay[QQ];
#pragma unroll
        for (int u = 0; u < QQ; ++u) ax[u] = ay[u] = 0.0;
        int j = 0;
        for (; j + 4 <= m; j += 4) {
            double2 v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                v[t] = reinterpret_cast<const double2*>(in + static_cast<int64_t>(ld_uniform_i(idx_in, j + t)) * n)[i2];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int u = 0; u < QQ; ++u) {
                    const double y = ld_uniform(Y, static_cast<int64_t>(j + t) * q + (u < q ? u : 0));
                    const double px = y * v[t].x;
                    const double py = y * v[t].y;
                    ax[u] = ax[u] + px;
                    ay[u] = ay[u] + py;
                }
            }
        }
        for (; j < m; ++j) {
            const double2 v = reinterpret_cast<const double2*>(in + static_cast<int64_t>(ld_uniform_i(idx_in, j)) * n)[i2];
#pragma unroll
            for (int u = 0; u < QQ; ++u) {
                const double y = ld_uniform(Y, static_cast<int64_t>(j) * q + (u < q ? u : 0));
                const double px = y * v.x;
                const double py = y * v.y;
                ax[u] = ax[u] + px;
                ay[u] = ay[u] + py;
            }
        }
#pragma unroll
        for (int u = 0; u < QQ; ++u) {
            if (u < q)
                reinterpret_cast<double2*>(out + static_cast<int64_t>(ld_uniform_i(idx_out, u)) * n)[i2] =
                    double2{ax[u], ay[u]};
            const double tx = ax[u] * ax[u];
            const double ty = ay[u] * ay[u];
            nrm[u] = nrm[u] + tx;
            nrm[u] = nrm[u] + ty;
        }
    }
    if (part) {
#pragma unroll
        for (int u = 0; u < QQ; ++u) {
            const double sv = block_sum(nrm[u], s_red);
            if (threadIdx.x == 0 && u < q) part[static_cast<int64_t>(blockIdx.x) * q + u] = sv;
        }
    }
}

// Two combinations in one pass over the inputs, on pairs of rows as in k_blk_comb2:
// out[c] = sum_{j < m} Y[j][c] in[j] and out2[c] = sum_{j0 <= j < m} Y[j][c] in[j]
// (c < q), each sum in ascending j from its own first term, so each equals what a pass
// of its own gives.  The Ritz step's X = S Y with P = S[j0:] Y[j0:].
template <int QQ>
__global__ __launch_bounds__(kBlock) void k_blk_comb2d(const double* __restrict__ in,
                                                       const int32_t* __restrict__ idx_in, int m, int j0,
                                                       const double* __restrict__ Y, double* __restrict__ out,
                                                       const int32_t* __restrict__ idx_out,
                                                       const int32_t* __restrict__ idx_out2, int q, int64_t n)
{
    const int64_t n2 = n >> 1;
    for (int64_t i2 = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i2 < n2;
         i2 += static_cast<int64_t>(gridDim.x) * kBlock) {
        double ax[QQ], ay[QQ], bx[QQ], by[QQ];
#pragma unroll
        for (int u = 0; u < QQ; ++u) ax[u] = ay[u] = bx[u] = by[u] = 0.0;
        // terms of inputs j .. j + G - 1 (G = 4 or 1); BOTH: they enter the second sum too
        auto terms = [&](int j, auto group, auto both) __attribute__((always_inline)) {
            constexpr int G = decltype(group)::value;
            double2 v[G];
#pragma unroll
            for (int t = 0; t < G; ++t)
                v[t] = reinterpret_cast<const double2*>(in + static_cast<int64_t>(ld_uniform_i(idx_in, j + t)) * n)[i2];
#pragma unroll
            for (int t = 0; t < G; ++t) {
#pragma unroll
                for (int u = 0; u < QQ; ++u) {
                    const double y = ld_uniform(Y, static_cast<int64_t>(j + t) * q + (u < q ? u : 0));
                    const double px = y * v[t].x;
                    const double py = y * v[t].y;
                    ax[u] = ax[u] + px;
                    ay[u] = ay[u] + py;
                    if constexpr (decltype(both)::value) {
                        bx[u] = bx[u] + px;
                        by[u] = by[u] + py;
                    }
                }
            }
        };
        using Four = std::integral_constant<int, 4>;
        using One = std::integral_constant<int, 1>;
        int j = 0;
        for (; j + 4 <= j0; j += 4) terms(j, Four{}, std::false_type{});
        for (; j < j0; ++j) terms(j, One{}, std::false_type{});
        for (; j + 4 <= m; j += 4) terms(j, Four{}, std::true_type{});
        for (; j < m; ++j) terms(j, One{}, std::true_type{});
#pragma unroll
        for (int u = 0; u < QQ; ++u)
            if (u < q) {
                reinterpret_cast<double2*>(out + static_cast<int64_t>(ld_uniform_i(idx_out, u)) * n)[i2] =
                    double2{ax[u], ay[u]};
                reinterpret_cast<double2*>(out + static_cast<int64_t>(ld_uniform_i(idx_out2, u)) * n)[i2] =
                    double2{bx[u], by[u]};
            }
    }
}

#undef LZ_ROWS

// Hellmann-Feynman gradient on the stored entries: gvals[e] = sum_r g[r] U[r][i] U[r][c]
// for entry e = (i, c), r ascending, each product rounded.  Tile of kTile rows per
// workgroup, entries walked as in k_pattern_outer.
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_eig_grad(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                                     const double* __restrict__ U, const double* __restrict__ g,
                                                     int k, int64_t n, double* __restrict__ gvals)
{
    __shared__ int64_t s_rp[kTile + 1];
    const int tid = threadIdx.x;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kTile;
    const int nr = static_cast<int>(min(static_cast<int64_t>(kTile), n - row0));
    for (int j = tid; j <= nr; j += kBlock) s_rp[j] = ld_rp(rp, row0 + j);
    __syncthreads();
    const int64_t k0 = s_rp[0], k1 = s_rp[nr];
    for (int64_t kk = k0 + tid; kk < k1; kk += kBlock) {
        int lo = 0, hi = nr;   // s_rp[lo] <= kk < s_rp[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_rp[mid] <= kk) lo = mid;
            else hi = mid;
        }
        const int64_t i = row0 + lo, c = col[kk];
        double acc = 0.0;
        for (int r = 0; r < k; ++r) {
            const double t = U[static_cast<int64_t>(r) * n + i] * U[static_cast<int64_t>(r) * n + c];
            const double t2 = g[r] * t;
            acc = acc + t2;
        }
        gvals[kk] = acc;
    }
}

// SparseTensorList packing: one item's pattern into the block-diagonal packed pattern
// (the pages' second batching mode, distinct patterns per item: paperpeel page, section
// 3.1 "Typed sparse-tensor hierarchy").
template <typename RPI, typename RPO>
__global__ __launch_bounds__(kBlock) void k_pack_pattern(const RPI* __restrict__ rp, const int32_t* __restrict__ col,
                                                         int64_t n, int64_t nnz, int64_t r0, int64_t e0,
                                                         int64_t rows_padded, RPO* __restrict__ out_rp,
                                                         int32_t* __restrict__ out_col)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    // rows r0 .. r0 + rows_padded inclusive: the last value (e0 + nnz) is also the next
    // item's first, written the same by both
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i <= rows_padded; i += stride)
        out_rp[r0 + i] = static_cast<RPO>(e0 + (i <= n ? static_cast<int64_t>(rp[i]) : nnz));
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; e < nnz; e += stride)
        out_col[e0 + e] = static_cast<int32_t>(r0 + col[e]);
}

// ----------------------------------------------------------------------------------
// Grouped batch (shared-pattern batches on unstructured patterns).  kGroup systems
// are interleaved element by element: vectors [group][n][kGroup], values
// [group][nnz][kGroup].  Lane t works on row t / kGroup of its tile for system
// t % kGroup, so one gathered element of all kGroup systems is one 32-byte piece of
// a cache line: the random gathers cost one cache request per kGroup systems instead
// of one per system.  Every lane sums its row in ascending entry order with rounded
// products, as the other SpMV kernels do, and the elementwise steps use the same
// expressions, so each system follows the same arithmetic as on its own.
// Grid (P, groups); with groups % 8 == 0 every group runs on one XCD (workgroup b
// runs on XCD b % 8), so the XCD's L2 holds that group's operand.
// ----------------------------------------------------------------------------------
constexpr int kGRows = kBlock / kGroup;   // rows per tile

struct GroupCoord {
    int grp;
    int lb;
};

__device__ __forceinline__ GroupCoord group_coord(const CgArgs& a, int P)
{
    if (a.groups >= 8 && (a.groups & 7) == 0) {
        const int64_t L = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
        const int x = static_cast<int>(L & 7);
        const int64_t slot = L >> 3;
        return GroupCoord{x + 8 * static_cast<int>(slot / P), static_cast<int>(slot % P)};
    }
    return GroupCoord{static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.x)};
}

// Per-system sum over the workgroup: lane t contributes v to system t % kGroup; every
// lane gets its system's total.  Fixed order (deterministic).  s_red: 4 * kGroup doubles.
__device__ __forceinline__ double group_block_sum(double v, double* s_red)
{
#pragma unroll
    for (int off = 32; off >= kGroup; off >>= 1) v = v + __shfl_xor(v, off, 64);
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    if (lane < kGroup) s_red[w * kGroup + lane] = v;
    __syncthreads();
    const int sy = threadIdx.x % kGroup;
    const double t = (s_red[sy] + s_red[kGroup + sy]) + (s_red[2 * kGroup + sy] + s_red[3 * kGroup + sy]);
    __syncthreads();
    return t;
}

// Per-system maximum over the workgroup (as group_block_sum, with max).
__device__ __forceinline__ double group_block_max(double v, double* s_red)
{
#pragma unroll
    for (int off = 32; off >= kGroup; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    if (lane < kGroup) s_red[w * kGroup + lane] = v;
    __syncthreads();
    const int sy = threadIdx.x % kGroup;
    const double t = fmax(fmax(s_red[sy], s_red[kGroup + sy]), fmax(s_red[2 * kGroup + sy], s_red[3 * kGroup + sy]));
    __syncthreads();
    return t;
}

// Per-system sum of the P partials part[sys][P] of the group's systems.
__device__ __forceinline__ double group_reduce_partials(const double* part, int sys0, int P, double* s_red)
{
    const int sy = threadIdx.x % kGroup;
    double v = 0.0;
    for (int j = threadIdx.x / kGroup; j < P; j += kBlock / kGroup)
        v = v + part[static_cast<int64_t>(sys0 + sy) * P + j];
    return group_block_sum(v, s_red);
}

// cg_step_begin for the group's systems: each lane decides for system sys0 + t % kGroup
// (the lane t < kGroup of workgroup 0 writes that system's records).  s_stop[kGroup]
// receives the stop words read at entry.  Contains barriers.
__device__ __forceinline__ int group_step_begin(const CgArgs& a, int sys0, int lb, int64_t k, double* s_red,
                                                int64_t* s_stop, double& beta, double& alpha_prev)
{
    const int sy = threadIdx.x % kGroup;
    const int sys = sys0 + sy;
    SysState* st = a.st + sys;
    const bool lead = (lb == 0 && threadIdx.x < kGroup);
    const bool first = (k == 0);
    if (threadIdx.x < kGroup) s_stop[threadIdx.x] = a.st[sys0 + threadIdx.x].stop_iter;
    const double rho_k = group_reduce_partials(a.part_rho, sys0, a.Gu, s_red);
    // |r_k|: from rho_k, or (Jacobi, rho_k = r^T z) from its own partials
    const double rr_k = a.jacobi ? group_reduce_partials(a.part_rr, sys0, a.Gu, s_red) : rho_k;
    const double diag_flags = (a.jacobi && first) ? group_reduce_partials(a.part_aux, sys0, a.Gu, s_red) : 0.0;
    beta = 0.0;
    alpha_prev = 0.0;
    if (s_stop[sy] < k) return kStepStopped;
    const double res = sqrt(rr_k);
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
    alpha_prev = first ? 0.0 : st->alpha[(k - 1) & 1];
    int code = -1;
    if (!a.fixed && res <= thr) code = SLA_CONVERGED;
    else if (diag_flags >= kDiagNaN) code = SLA_NAN;        // Jacobi, k = 0: unusable diagonal
    else if (diag_flags > 0.0) code = SLA_NOT_SPD;
    else if (k >= a.max_iter) code = SLA_MAX_ITER;
    if (code >= 0) {
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
        return kStepStopNow;
    }
    beta = first ? 0.0 : rho_k / st->rho[(k - 1) & 1];
    if (lead) {
        st->rho[k & 1] = rho_k;
        st->rr = rr_k;
        if (first) { st->thr = thr; st->rhs = rhs; }
    }
    return kStepRun;
}

__device__ __forceinline__ bool group_any_running(const int64_t* s_stop, int64_t after)
{
    bool any = false;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) any = any || (s_stop[j] > after);
    return any;
}

// Grouped layout of the values: out[g][k][s] = vals[g * kGroup + s][k].
__global__ __launch_bounds__(kBlock) void k_group_vals(const double* __restrict__ vals, double* __restrict__ out,
                                                       int64_t nnz, int groups, const int32_t* __restrict__ eperm)
{
    const int64_t total = nnz * kGroup;
    const int g = blockIdx.y;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * kBlock) {
        const int64_t kk = e / kGroup;
        const int sy = static_cast<int>(e - kk * kGroup);
        const int64_t src = eperm ? static_cast<int64_t>(eperm[kk]) : kk;   // reordered pattern: old entry
        out[static_cast<int64_t>(g) * total + e] = vals[(static_cast<int64_t>(g) * kGroup + sy) * nnz + src];
    }
}

// x = 0, p_{-1} = 0, r_0 = b (into the grouped layout), partial r_0^T r_0, state reset.
__global__ __launch_bounds__(kBlock) void k_gcg_init(CgArgs a)
{
    __shared__ double s_red[4 * kGroup];
    const GroupCoord gc = group_coord(a, a.Gu);
    const int tid = threadIdx.x;
    const int sy = tid % kGroup;
    const int sys0 = gc.grp * kGroup;
    const int64_t n = a.n;
    const int64_t goff = static_cast<int64_t>(gc.grp) * n * kGroup;
    const double* __restrict__ b = a.b + static_cast<int64_t>(sys0 + sy) * n;
    const int64_t gtiles = (n + kGRows - 1) / kGRows;
    const bool jac = a.jacobi != 0;
    double rr = 0.0, rz = 0.0;
    for (int64_t t = gc.lb; t < gtiles; t += a.Gu) {
        const int64_t i = t * kGRows + tid / kGroup;
        if (i < n) {
            const int64_t e = goff + i * kGroup + sy;
            const double bv = b[a.gperm ? a.gperm[i] : i];   // reordered pattern: row i was row gperm[i]
            a.r[e] = bv;
            a.xg[e] = 0.0;
            a.p1[e] = 0.0;
            const double w = bv * bv;
            rr = rr + w;
            if (jac) {                       // z_0 = M^{-1} b
                const double zv = bv / a.dg[e];
                a.z[e] = zv;
                const double wz = bv * zv;
                rz = rz + wz;
            }
        }
    }
    rr = group_block_sum(rr, s_red);
    if (jac) rz = group_block_sum(rz, s_red);
    if (tid < kGroup) {
        const int64_t slot = static_cast<int64_t>(sys0 + tid) * a.Gu + gc.lb;
        if (jac) {
            a.part_rr[slot] = rr;
            a.part_rho[slot] = rz;
        } else {
            a.part_rho[slot] = rr;
        }
        if (gc.lb == 0) a.st[sys0 + tid].stop_iter = INT64_MAX;
    }
    if (gc.lb == 0 && gc.grp == 0 && tid == 0) *a.n_active = a.batch;
}

// The step's decisions, p_k = r_k + beta p_{k-1} and x_k = x_{k-1} + alpha_{k-1} p_{k-1}.
__global__ __launch_bounds__(kBlock) void k_gcg_pupd(CgArgs a, int64_t k)
{
    __shared__ double s_red[4 * kGroup];
    __shared__ int64_t s_stop[kGroup];
    const GroupCoord gc = group_coord(a, a.Gu);
    const int tid = threadIdx.x;
    const int sy = tid % kGroup;
    const int sys0 = gc.grp * kGroup;
    double beta, alpha_prev;
    const int run = group_step_begin(a, sys0, gc.lb, k, s_red, s_stop, beta, alpha_prev);
    if (!group_any_running(s_stop, k - 1)) return;   // every system stopped earlier
    if (run == kStepStopped || (run == kStepStopNow && k == 0)) return;
    const bool stop = (run == kStepStopNow);
    const int64_t n = a.n;
    const int64_t goff = static_cast<int64_t>(gc.grp) * n * kGroup;
    const double* __restrict__ rg = (a.jacobi ? a.z : a.r) + goff;   // p_k = z_k + beta p_{k-1} with Jacobi
    const double* __restrict__ pp = ((k & 1) ? a.p0 : a.p1) + goff;
    double* __restrict__ pc = ((k & 1) ? a.p1 : a.p0) + goff;
    double* __restrict__ xg = a.xg + goff;
    const int64_t gtiles = (n + kGRows - 1) / kGRows;
    (void)sy;
#pragma unroll 1
    for (int64_t t0 = gc.lb; t0 < gtiles; t0 += kStreamUnroll * static_cast<int64_t>(a.Gu)) {
        double rv[kStreamUnroll], pv[kStreamUnroll], xv[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t i = min((t0 + u * static_cast<int64_t>(a.Gu)) * kGRows + tid / kGroup, n - 1);
            const int64_t e = i * kGroup + tid % kGroup;
            rv[u] = rg[e];
            pv[u] = pp[e];
            xv[u] = xg[e];
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t t = t0 + u * static_cast<int64_t>(a.Gu);
            const int64_t i = t * kGRows + tid / kGroup;
            if (t < gtiles && i < n) {
                const int64_t e = i * kGroup + tid % kGroup;
                const double tx = alpha_prev * pv[u];
                xg[e] = xv[u] + tx;
                if (!stop) {
                    const double tp = beta * pv[u];
                    pc[e] = rv[u] + tp;
                }
            }
        }
    }
}

// q = A p_k for the group's systems (p_k formed by k_gcg_pupd), partial p_k^T q.
// Tiles of kGRows rows: the tile's entries (values of all kGroup systems, columns) are
// one contiguous range, loaded coalesced and staged through LDS (the lanes of one row
// read its entries there).  Pipelined like the banded kernel: while tile t is summed,
// the next tile's loads are in flight, every load unconditional (clamped), and the
// outputs are stored after the next commit.
//
// The operand, two ways:
//   * WIN = false: workgroup lb takes tiles lb, lb + P, ... and gathers p_k[col] of
//     every entry from memory (through the XCD's L2, which holds the group's operand);
//   * WIN = true (a pattern whose bandwidth, after the reordering, is at most
//     kGWinMaxHalo rows): workgroup lb takes one contiguous run of tiles and keeps an
//     LDS ring of the operand rows [row0 - H, row0 + kGRows + H) of its current tile, H =
//     a.g_halo (a multiple of kGRows).  Every column of the tile's rows lies in that
//     range, so the gathers are LDS reads; moving to the next tile loads one coalesced
//     chunk of kGRows rows (all kGroup systems) into the ring, the chunk H rows past the
//     next tile.  The first tile of a run fills the ring with 2 H / kGRows + 1 chunks.
//     The columns come as 16-bit offsets from the tile's first row (every column lies
//     within H + kGRows - 1 of it).
// Both give the same row sums (same products, same order); they differ in which
// workgroup sums which rows, so the partials of p^T q are grouped differently.
template <int CAPG>   // entries per tile (kGRows rows of at most CAPG / kGRows entries)
struct GStage {
    double v[CAPG * kGroup / kBlock];
    int32_t c[CAPG / kBlock];
    int32_t a0, a1;
    double w;   // WIN: this lane's element of the operand chunk the next tile brings in
};

constexpr int kGWinRows = 1024;   // operand ring (rows; a power of two, a multiple of kGRows)
// Largest halo in chunks: a tile's 2 hc + 1 chunks must occupy distinct ring slots.
constexpr int kGWinHaloChunks = (kGWinRows / kGRows - 1) / 2;
static_assert(kGWinHaloChunks * kGRows == kGWinMaxHalo, "the host's window limit is the ring's");

template <int CAPG, bool WIN>
__global__ __launch_bounds__(kBlock) void k_gcg_spmv(CgArgs a, int64_t k)
{
    constexpr int UV = CAPG * kGroup / kBlock;
    constexpr int UC = CAPG / kBlock;
    constexpr int RC = 8;
    __shared__ double s_val[CAPG * kGroup];
    __shared__ int32_t s_col[CAPG];
    __shared__ int32_t s_rs[kBlock], s_re[kBlock];
    __shared__ double s_red[4 * kGroup];
    __shared__ int64_t s_stop[kGroup];
    __shared__ double s_win[WIN ? kGWinRows * kGroup : 1];
    const GroupCoord gc = group_coord(a, a.G);
    const int tid = threadIdx.x;
    const int sy = tid % kGroup;
    const int sys0 = gc.grp * kGroup;
    if (tid < kGroup) s_stop[tid] = a.st[sys0 + tid].stop_iter;
    __syncthreads();
    if (!group_any_running(s_stop, k)) return;   // k_gcg_pupd stopped all of them at k or before
    const bool run = s_stop[sy] > k;
    const int32_t n = static_cast<int32_t>(a.n);
    const int64_t goff = static_cast<int64_t>(gc.grp) * a.n * kGroup;
    const int32_t* __restrict__ rp = static_cast<const int32_t*>(a.row_ptr);
    const int32_t* __restrict__ col = a.col;
    const double* __restrict__ vg = a.vals + static_cast<int64_t>(gc.grp) * a.nnz * kGroup;
    const double* __restrict__ pg = ((k & 1) ? a.p1 : a.p0) + goff;
    double* __restrict__ qg = a.q + goff;
    const int32_t gtiles = (n + kGRows - 1) / kGRows;
    const int32_t P = a.G;
    const int32_t nnz = static_cast<int32_t>(a.nnz);
    // tiles of this workgroup: t = tb, tb + ts, ... while t < te
    const int32_t tb = WIN ? static_cast<int32_t>((static_cast<int64_t>(gc.lb) * gtiles) / P) : gc.lb;
    const int32_t te = WIN ? static_cast<int32_t>((static_cast<int64_t>(gc.lb + 1) * gtiles) / P) : gtiles;
    const int32_t ts = WIN ? 1 : P;
    const int32_t hc = WIN ? a.g_halo / kGRows : 0;   // halo chunks on each side
    auto tk0 = [&](int32_t t) { return static_cast<int32_t>(ld_rp_uniform(rp, min(t * kGRows, n))); };
    auto tk1 = [&](int32_t t) { return static_cast<int32_t>(ld_rp_uniform(rp, min((t + 1) * kGRows, n))); };
    // WIN: this lane's element of operand chunk c (rows c kGRows ...), clamped into range
    auto chunk_ld = [&](int32_t c) __attribute__((always_inline)) {
        const int32_t i = min(max(c * kGRows + tid / kGroup, 0), n - 1);
        return pg[static_cast<int64_t>(i) * kGroup + sy];
    };
    auto chunk_st = [&](int32_t c, double v) __attribute__((always_inline)) {
        const int32_t i = c * kGRows + tid / kGroup;   // may lie outside [0, n): never read then
        s_win[(i & (kGWinRows - 1)) * kGroup + sy] = v;
    };
    // issue the loads of tile t (entries [k0, k1)); clamped, so every lane issues them all
    auto stage = [&](GStage<CAPG>& S, int32_t t, int32_t k0, int32_t k1) __attribute__((always_inline)) {
        const int32_t i = min(t * kGRows + tid / kGroup, n - 1);
        S.a0 = rp[i];
        S.a1 = rp[i + 1];
        const int32_t cnt = k1 - k0;
        const int32_t kb = cnt > 0 ? k0 : min(k0, nnz - 1);
        const double* __restrict__ vb = vg + static_cast<int64_t>(kb) * kGroup;
        const int lastv = max(cnt * kGroup - 1, 0), lastc = max(cnt - 1, 0);
        // the values (every system's, read once per SpMV) stream with the non-temporal
        // hint, leaving the caches to the operand
#pragma unroll
        for (int u = 0; u < UV; ++u) S.v[u] = __builtin_nontemporal_load(vb + min(tid + u * kBlock, lastv));
        if constexpr (WIN) {
            // 16-bit offsets from the tile's first row (sign-extended by the load); the
            // commit adds the row back
            const int16_t* __restrict__ cb = a.g_col16 + kb;
#pragma unroll
            for (int u = 0; u < UC; ++u) S.c[u] = cb[min(tid + u * kBlock, lastc)];
            S.w = chunk_ld(t + hc);   // the chunk this tile adds to the ring
        } else {
            const int32_t* __restrict__ cb = col + kb;
#pragma unroll
            for (int u = 0; u < UC; ++u) S.c[u] = cb[min(tid + u * kBlock, lastc)];
        }
    };
    // Every staged register is written to LDS on every path (slots past the tile's
    // entries take the clamped loads' copies and are never read), so no load is left
    // unconsumed on a branch, which would make the compiler drain the loads in flight.
    auto commit = [&](const GStage<CAPG>& S, int32_t t, int32_t k0, int32_t k1) __attribute__((always_inline)) {
        (void)k1;
#pragma unroll
        for (int u = 0; u < UV; ++u) s_val[tid + u * kBlock] = S.v[u];
        const int32_t cbase = WIN ? t * kGRows : 0;
#pragma unroll
        for (int u = 0; u < UC; ++u) s_col[tid + u * kBlock] = S.c[u] + cbase;
        const bool has = t * kGRows + tid / kGroup < n;
        s_rs[tid] = S.a0 - k0;
        s_re[tid] = has ? S.a1 - k0 : S.a0 - k0;
        if constexpr (WIN) chunk_st(t + hc, S.w);
    };
    auto operand = [&](int32_t c) __attribute__((always_inline)) {
        if constexpr (WIN) return s_win[(c & (kGWinRows - 1)) * kGroup + sy];
        else return pg[static_cast<int64_t>(c) * kGroup + sy];
    };

    double sig = 0.0;
    int32_t t = tb;
    if (t >= te) {
        sig = group_block_sum(sig, s_red);
        if (tid < kGroup) a.part_sigma[static_cast<int64_t>(sys0 + tid) * a.G + gc.lb] = sig;
        return;
    }
    // Three stage buffers in rotation: while tile t is summed, tiles t + ts and t + 2 ts
    // are loading, so each tile's loads have two tile times to arrive (with one tile
    // ahead the kernel waited on memory once per tile).
    GStage<CAPG> SA, SB, SC;
    int32_t k0a = tk0(t), k1a = tk1(t), k0b = 0, k1b = 0, k0c = 0, k1c = 0;
    if (t + ts < te) {
        k0b = tk0(t + ts);
        k1b = tk1(t + ts);
    }
    stage(SA, t, k0a, k1a);
    if constexpr (WIN) {
        // the ring's first fill: chunks t - hc ... t + hc - 1 (the stages bring t + hc
        // and t + hc + 1), every load issued before the first store (unconditional: past
        // 2 hc they repeat the last chunk)
        double fill[2 * kGWinHaloChunks];
#pragma unroll
        for (int u = 0; u < 2 * kGWinHaloChunks; ++u) fill[u] = chunk_ld(t - hc + min(u, max(2 * hc - 1, 0)));
#pragma unroll
        for (int u = 0; u < 2 * kGWinHaloChunks; ++u)
            if (u < 2 * hc) chunk_st(t - hc + u, fill[u]);
    }
    if (t + 2 * ts < te) {
        k0c = tk0(t + 2 * ts);
        k1c = tk1(t + 2 * ts);
    }
    commit(SA, t, k0a, k1a);
    // staged after the first commit, so the loop starts with its loads the only ones in
    // flight
    stage(SB, t + ts, k0b, k1b);   // past the end: clamped loads
    __syncthreads();
    // stg: the buffer that takes tile t + 2 ts; cmt: the buffer holding tile t + ts
#define SLA_GCG_TILE(stg, cmt)                                                                             \
    {                                                                                                      \
        stage(stg, t + 2 * ts, k0c, k1c); /* past the end: clamped loads, keeps the wait counts exact */  \
        int32_t k0d = 0, k1d = 0;                                                                          \
        if (t + 3 * ts < te) {                                                                             \
            k0d = tk0(t + 3 * ts);                                                                         \
            k1d = tk1(t + 3 * ts);                                                                         \
        }                                                                                                  \
        const int rs = s_rs[tid], re = s_re[tid];                                                          \
        double sum = 0.0;                                                                                  \
        for (int j0 = rs; j0 < re; j0 += RC) {                                                             \
            double pv[RC];                                                                                 \
            _Pragma("unroll") for (int u = 0; u < RC; ++u) {                                               \
                const int j = (j0 + u < re) ? j0 + u : j0;                                                 \
                pv[u] = operand(s_col[j]);                                                                 \
            }                                                                                              \
            _Pragma("unroll") for (int u = 0; u < RC; ++u) {                                               \
                const bool ok = j0 + u < re;                                                               \
                const int j = ok ? j0 + u : j0;                                                            \
                const double tt = s_val[j * kGroup + sy] * pv[u];                                          \
                const double sn = sum + tt;                                                                \
                sum = ok ? sn : sum;                                                                       \
            }                                                                                              \
        }                                                                                                  \
        const int32_t i = t * kGRows + tid / kGroup;                                                       \
        const double pown = WIN ? operand(min(i, n - 1)) : 0.0;                                            \
        __syncthreads(); /* tile t's LDS reads are done */                                                 \
        t += ts;                                                                                           \
        const int32_t k0n = k0b, k1n = k1b;                                                                \
        k0b = k0c;                                                                                         \
        k1b = k1c;                                                                                         \
        k0c = k0d;                                                                                         \
        k1c = k1d;                                                                                         \
        /* unconditional (past the end it commits an empty tile nothing reads), so no */                \
        /* staged load is left unconsumed on a path                                   */                \
        commit(cmt, t, k0n, k1n);                                                                          \
        if (run && i < n) {                                                                                \
            const int64_t e = static_cast<int64_t>(i) * kGroup + sy;                                      \
            qg[e] = sum;                                                                                   \
            const double w = (WIN ? pown : pg[e]) * sum;                                                   \
            sig = sig + w;                                                                                 \
        }                                                                                                  \
        if (t >= te) break;                                                                                \
        __syncthreads();                                                                                   \
    }
#pragma unroll 1
    while (true) {
        SLA_GCG_TILE(SC, SB)
        SLA_GCG_TILE(SA, SC)
        SLA_GCG_TILE(SB, SA)
    }
#undef SLA_GCG_TILE
    sig = group_block_sum(sig, s_red);
    if (tid < kGroup) a.part_sigma[static_cast<int64_t>(sys0 + tid) * a.G + gc.lb] = sig;
}

// alpha = rho / sigma per system, r -= alpha q, partial r^T r.
__global__ __launch_bounds__(kBlock) void k_gcg_update(CgArgs a, int64_t k)
{
    __shared__ double s_red[4 * kGroup];
    __shared__ int64_t s_stop[kGroup];
    const GroupCoord gc = group_coord(a, a.Gu);
    const int tid = threadIdx.x;
    const int sy = tid % kGroup;
    const int sys0 = gc.grp * kGroup;
    const int sys = sys0 + sy;
    SysState* st = a.st + sys;
    if (tid < kGroup) s_stop[tid] = a.st[sys0 + tid].stop_iter;
    const double sigma = group_reduce_partials(a.part_sigma, sys0, a.G, s_red);
    if (!group_any_running(s_stop, k)) return;
    bool run = s_stop[sy] > k;
    const double rho_k = st->rho[k & 1];
    if (run && !(sigma > 0.0)) {
        if (gc.lb == 0 && tid < kGroup) {
            st->stop_iter = k;
            sla_cg_info inf;
            inf.iterations = k;
            inf.res_norm = sqrt(a.jacobi ? st->rr : rho_k);
            inf.rhs_norm = st->rhs;
            inf.state = (sigma != sigma) ? SLA_NAN : SLA_NOT_SPD;
            inf.reserved = 0;
            a.info[sys] = inf;
            atomicSub(a.n_active, 1);
        }
        run = false;
    }
    const double alpha = rho_k / sigma;
    if (run && gc.lb == 0 && tid < kGroup) st->alpha[k & 1] = alpha;
    const int64_t n = a.n;
    const int64_t goff = static_cast<int64_t>(gc.grp) * n * kGroup;
    const double* __restrict__ qg = a.q + goff;
    double* __restrict__ rg = a.r + goff;
    const bool jac = a.jacobi != 0;
    const double* __restrict__ dgg = jac ? a.dg + goff : nullptr;
    double* __restrict__ zg = jac ? a.z + goff : nullptr;
    const int64_t gtiles = (n + kGRows - 1) / kGRows;
    double rr = 0.0, rz = 0.0;
    if (run) {
#pragma unroll 1
        for (int64_t t0 = gc.lb; t0 < gtiles; t0 += kStreamUnroll * static_cast<int64_t>(a.Gu)) {
            double qv[kStreamUnroll], rv[kStreamUnroll];
#pragma unroll
            for (int u = 0; u < kStreamUnroll; ++u) {
                const int64_t i = min((t0 + u * static_cast<int64_t>(a.Gu)) * kGRows + tid / kGroup, n - 1);
                const int64_t e = i * kGroup + sy;
                qv[u] = qg[e];
                rv[u] = rg[e];
            }
#pragma unroll
            for (int u = 0; u < kStreamUnroll; ++u) {
                const int64_t t = t0 + u * static_cast<int64_t>(a.Gu);
                const int64_t i = t * kGRows + tid / kGroup;
                if (t < gtiles && i < n) {
                    const double tq = alpha * qv[u];
                    const double rn = rv[u] - tq;
                    rg[i * kGroup + sy] = rn;
                    const double w = rn * rn;
                    rr = rr + w;
                    if (jac) {
                        const double zn = rn / dgg[i * kGroup + sy];   // z = M^{-1} r
                        zg[i * kGroup + sy] = zn;
                        const double wz = rn * zn;
                        rz = rz + wz;
                    }
                }
            }
        }
    }
    rr = group_block_sum(rr, s_red);
    if (jac) rz = group_block_sum(rz, s_red);
    if (tid < kGroup) {
        const int64_t slot = static_cast<int64_t>(sys0 + tid) * a.Gu + gc.lb;
        if (jac) {
            a.part_rr[slot] = rr;
            a.part_rho[slot] = rz;
        } else {
            a.part_rho[slot] = rr;
        }
    }
}

// Jacobi: the diagonal in the grouped layout (entry (i, i) by binary search in row i of
// the shared 32-bit pattern; 0 if not stored) and the flag partials of k_cg_diag.
__global__ __launch_bounds__(kBlock) void k_gcg_diag(CgArgs a)
{
    __shared__ double s_red[4 * kGroup];
    const GroupCoord gc = group_coord(a, a.Gu);
    const int tid = threadIdx.x;
    const int sy = tid % kGroup;
    const int sys0 = gc.grp * kGroup;
    const int64_t n = a.n;
    const int64_t goff = static_cast<int64_t>(gc.grp) * n * kGroup;
    const int32_t* __restrict__ rp = static_cast<const int32_t*>(a.row_ptr);
    const double* __restrict__ vg = a.vals + static_cast<int64_t>(gc.grp) * a.nnz * kGroup;
    const int64_t gtiles = (n + kGRows - 1) / kGRows;
    double flag = 0.0;
    for (int64_t t = gc.lb; t < gtiles; t += a.Gu) {
        const int64_t i = t * kGRows + tid / kGroup;
        if (i < n) {
            int64_t lo = rp[i], hi = rp[i + 1];
            const int64_t end = hi;
            while (lo < hi) {
                const int64_t mid = (lo + hi) >> 1;
                if (a.col[mid] < i) lo = mid + 1;
                else hi = mid;
            }
            const double d = (lo < end && a.col[lo] == i) ? vg[lo * kGroup + sy] : 0.0;
            a.dg[goff + i * kGroup + sy] = d;
            if (d != d) flag = kDiagNaN;
            else if (!(d > 0.0)) flag = fmax(flag, kDiagNonPos);
        }
    }
    flag = group_block_max(flag, s_red);
    if (tid < kGroup) a.part_aux[static_cast<int64_t>(sys0 + tid) * a.Gu + gc.lb] = flag;
}

// x[s][i] = xg[i][s]: the solutions back in the caller's layout (and order).
__global__ __launch_bounds__(kBlock) void k_gcg_finish(CgArgs a)
{
    const GroupCoord gc = group_coord(a, a.Gu);
    const int tid = threadIdx.x;
    const int sy = tid % kGroup;
    const int64_t n = a.n;
    const int64_t goff = static_cast<int64_t>(gc.grp) * n * kGroup;
    double* __restrict__ x = a.x + static_cast<int64_t>(gc.grp * kGroup + sy) * n;
    const int64_t gtiles = (n + kGRows - 1) / kGRows;
    for (int64_t t = gc.lb; t < gtiles; t += a.Gu) {
        const int64_t i = t * kGRows + tid / kGroup;
        if (i < n) x[a.gperm ? a.gperm[i] : i] = a.xg[goff + i * kGroup + sy];
    }
}

// ----------------------------------------------------------------------------------
// y = A x (one tile per workgroup; grid (ntiles, batch))
// ----------------------------------------------------------------------------------
template <typename RP, int CAP, bool OFF32>
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
    GatherX<OFF32> g{x + static_cast<int64_t>(sys) * n_cols};
    const double s = tile_rowsum<RP, CAP, row_chunk(CAP)>(rp, col, vals + static_cast<int64_t>(sys) * nnz, row0,
                                                          nr, g, s_val, s_col);
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
__device__ __forceinline__ int32_t wave_max_i32(int32_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ int32_t wave_min_i32(int32_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
    return v;
}

// Grid-stride over 256-row tiles; each workgroup folds its maxima / minima in
// registers and LDS and issues one atomic per counter at the end (a per-row or
// per-tile atomic on one address serialises at the L2 for large patterns).
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_validate(const RP* __restrict__ rp, const int32_t* __restrict__ col,
                                                     int64_t n_rows, int64_t n_cols, int64_t nnz, int32_t* out)
{
    __shared__ int32_t s_m[3][kBlock / 64];
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid == 0) {
        if (ld_rp(rp, 0) != 0 || ld_rp(rp, n_rows) != nnz) atomicOr(out + kChkErr, 1);
    }
    const int64_t ntiles = (n_rows + kTile - 1) / kTile;
    int32_t err = 0, row_len = 0, far_min = 0x7fffffff, far_max = 0, tile_max = 0;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t i = t * kTile + tid;
        if (i < n_rows) {
            const int64_t a = ld_rp(rp, i), e = ld_rp(rp, i + 1);
            if (a > e || a < 0 || e > nnz) {
                err |= 2;
            } else {
                int64_t prev = -1;
                for (int64_t kk = a; kk < e; ++kk) {
                    const int64_t c = col[kk];
                    if (c < 0 || c >= n_cols) err |= 4;
                    if (c <= prev) err |= 8;
                    prev = c;
                    const int64_t d = min(c > i ? c - i : i - c, int64_t(0x7fffffff));
                    if (d > kBandHalo) {
                        far_min = min(far_min, static_cast<int32_t>(d));
                        far_max = max(far_max, static_cast<int32_t>(d));
                    }
                }
                row_len = max(row_len, static_cast<int32_t>(min(e - a, int64_t(0x7fffffff))));
            }
            if (tid == 0) {
                const int64_t last = min(i + kTile, n_rows);
                const int64_t cnt = ld_rp(rp, last) - a;
                if (cnt > 0) tile_max = max(tile_max, static_cast<int32_t>(min(cnt, int64_t(0x7fffffff))));
            }
        }
    }
    if (err) atomicOr(out + kChkErr, err);
    row_len = wave_max_i32(row_len);
    far_min = wave_min_i32(far_min);
    far_max = wave_max_i32(far_max);
    const int w = tid >> 6;
    if ((tid & 63) == 0) {
        s_m[0][w] = row_len;
        s_m[1][w] = far_min;
        s_m[2][w] = far_max;
    }
    __syncthreads();
    if (tid == 0) {
        for (int v = 1; v < kBlock / 64; ++v) {
            row_len = max(row_len, s_m[0][v]);
            far_min = min(far_min, s_m[1][v]);
            far_max = max(far_max, s_m[2][v]);
        }
        if (row_len > 0) atomicMax(out + kChkRowMax, row_len);
        if (far_max > 0) {
            atomicMin(out + kChkFarMin, far_min);
            atomicMax(out + kChkFarMax, far_max);
        }
        if (tile_max > 0) atomicMax(out + kChkTileMax, tile_max);
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

// out[e] = col[e] - (first row of e's 256-row tile): one workgroup per tile, whose
// entries are contiguous.  The caller has checked that every offset fits 16 bits.
__global__ __launch_bounds__(kBlock) void k_col16(const int32_t* __restrict__ rp, const int32_t* __restrict__ col,
                                                  int16_t* __restrict__ out, int64_t n)
{
    const int64_t ntiles = (n + kTile - 1) / kTile;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t row0 = t * kTile;
        const int64_t k0 = rp[row0], k1 = rp[min(row0 + kTile, n)];
        for (int64_t e = k0 + threadIdx.x; e < k1; e += kBlock)
            out[e] = static_cast<int16_t>(col[e] - static_cast<int32_t>(row0));
    }
}

// out[e] = col[e] - (first row of the banded SpMV's window holding e's row i: line
// i / S, strip (i % S) / kTile): one thread per row.  The caller has checked that S
// fits (every offset lies in [-S, S + kTile - 1]).
__global__ __launch_bounds__(kBlock) void k_colb16(const int32_t* __restrict__ rp, const int32_t* __restrict__ col,
                                                   int16_t* __restrict__ out, int64_t n, int32_t S)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        const int32_t ii = static_cast<int32_t>(i);
        const int32_t wb = (ii / S) * S + ((ii % S) / kTile) * kTile;
        for (int32_t e = rp[i]; e < rp[i + 1]; ++e) out[e] = static_cast<int16_t>(col[e] - wb);
    }
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

using CgKernel = void (*)(CgArgs, int64_t);

template <typename RP, bool O, int MODE, bool C16 = false>
CgKernel spmv_kernel_rp(int cap)
{
    if (cap <= kCapSmall) return k_cg_spmv<RP, kCapSmall, O, MODE, C16>;
    if (cap <= kCapMid) return k_cg_spmv<RP, kCapMid, O, MODE, C16>;
    if (cap == kCapSkew) return k_cg_spmv<RP, kCapSkew, O, MODE, C16>;
    return k_cg_spmv<RP, kCapLarge, O, MODE, C16>;
}

// c16: the 16-bit column offsets (built only with 32-bit row pointers and n < 2^29).
template <int MODE>
CgKernel spmv_kernel_mode(int rp_bits, int cap, bool off32, bool c16 = false)
{
    if (c16 && rp_bits == 32 && off32) return spmv_kernel_rp<int32_t, true, MODE, true>(cap);
    if (rp_bits == 64)
        return off32 ? spmv_kernel_rp<int64_t, true, MODE>(cap) : spmv_kernel_rp<int64_t, false, MODE>(cap);
    return off32 ? spmv_kernel_rp<int32_t, true, MODE>(cap) : spmv_kernel_rp<int32_t, false, MODE>(cap);
}

CgKernel spmv_kernel(int rp_bits, int cap, bool off32, bool split = false, bool c16 = false)
{
    return split ? spmv_kernel_mode<kSpmvSplit>(rp_bits, cap, off32, c16)
                 : spmv_kernel_mode<kSpmvFused>(rp_bits, cap, off32, c16);
}

inline bool off32_ok(int64_t n) { return n < (int64_t(1) << 29); }

// c16: the window-relative 16-bit column offsets (a.col16 of a banded solve)
CgKernel band_kernel(int cap, bool c16 = false)
{
    if (c16) {
        if (cap <= kCapSmall) return k_cg_spmv_band<kCapSmall, true>;
        if (cap <= kCapMid) return k_cg_spmv_band<kCapMid, true>;
        return k_cg_spmv_band<kCapLarge, true>;
    }
    if (cap <= kCapSmall) return k_cg_spmv_band<kCapSmall, false>;
    if (cap <= kCapMid) return k_cg_spmv_band<kCapMid, false>;
    return k_cg_spmv_band<kCapLarge, false>;
}

template <typename RP, bool O>
hipError_t launch_matvec_rp(const RP* rp, const int32_t* col, const double* vals, const double* x, double* y,
                            int64_t n_rows, int64_t nnz, int64_t n_cols, int batch, int cap, hipStream_t s)
{
    const int64_t ntiles = (n_rows + kTile - 1) / kTile;
    const dim3 grid(static_cast<unsigned>(ntiles), batch), block(kBlock);
    if (cap <= kCapSmall)
        SLA_LAUNCH((k_matvec<RP, kCapSmall, O>), grid, block, 0, s, rp, col, vals, x, y, n_rows, nnz, n_cols);
    else if (cap <= kCapMid)
        SLA_LAUNCH((k_matvec<RP, kCapMid, O>), grid, block, 0, s, rp, col, vals, x, y, n_rows, nnz, n_cols);
    else if (cap == kCapSkew)
        SLA_LAUNCH((k_matvec<RP, kCapSkew, O>), grid, block, 0, s, rp, col, vals, x, y, n_rows, nnz, n_cols);
    else
        SLA_LAUNCH((k_matvec<RP, kCapLarge, O>), grid, block, 0, s, rp, col, vals, x, y, n_rows, nnz, n_cols);
    return hipGetLastError();
}

template <typename RP>
hipError_t launch_matvec_any(const RP* rp, const int32_t* col, const double* vals, const double* x, double* y,
                             int64_t n_rows, int64_t nnz, int64_t n_cols, int batch, int cap, hipStream_t s)
{
    if (off32_ok(n_cols))
        return launch_matvec_rp<RP, true>(rp, col, vals, x, y, n_rows, nnz, n_cols, batch, cap, s);
    return launch_matvec_rp<RP, false>(rp, col, vals, x, y, n_rows, nnz, n_cols, batch, cap, s);
}

}  // namespace

// ----------------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------------
int cg_blocks_per_cu(int rp_bits, int cap, int64_t n, bool split)
{
    static int cache[2][4][2][2] = {};   // occupancy is fixed per variant: query once
    const int ri = rp_bits == 64 ? 1 : 0;
    const int ci = cap <= kCapSmall ? 0 : (cap <= kCapMid ? 1 : (cap == kCapSkew ? 3 : 2));
    const bool o = off32_ok(n);
    int& c = cache[ri][ci][o ? 1 : 0][split ? 1 : 0];
    if (c > 0) return c;
    int a = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, spmv_kernel(rp_bits, cap, o, split), kBlock, 0) !=
            hipSuccess ||
        a < 1)
        a = 1;
    c = a;
    return c;
}

int cg_band_blocks_per_cu(int cap)
{
    static int cache[3] = {};
    int& c = cache[cap <= kCapSmall ? 0 : (cap <= kCapMid ? 1 : 2)];
    if (c > 0) return c;
    int a = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, band_kernel(cap), kBlock, 0) != hipSuccess || a < 1) a = 1;
    c = a;
    return c;
}

int cg_group_blocks_per_cu(int cap, bool win)
{
    static int cache[2][2] = {};
    int& c = cache[cap <= kGCapSmall ? 0 : 1][win ? 1 : 0];
    if (c > 0) return c;
    CgKernel f = cap <= kGCapSmall ? (win ? k_gcg_spmv<kGCapSmall, true> : k_gcg_spmv<kGCapSmall, false>)
                                   : (win ? k_gcg_spmv<kGCapLarge, true> : k_gcg_spmv<kGCapLarge, false>);
    int a = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, f, kBlock, 0) != hipSuccess || a < 1) a = 1;
    c = a;
    return c;
}

hipError_t launch_cg_diag(const CgArgs& a, int rp_bits, hipStream_t s)
{
    if (rp_bits == 64) SLA_LAUNCH(k_cg_diag<int64_t>, dim3(a.Gu, a.batch), dim3(kBlock), 0, s, a);
    else SLA_LAUNCH(k_cg_diag<int32_t>, dim3(a.Gu, a.batch), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_cg_init(const CgArgs& a, hipStream_t s)
{
    SLA_LAUNCH(k_cg_init, dim3(a.Gu, a.batch), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

// The diagonal-layout SpMV for nd diagonals: 5, 8 or 16 slots, 8-bit masks up to 8.
CgKernel dia_kernel(int nd)
{
    if (nd <= 5) return k_cg_spmv_dia<5, false>;
    if (nd <= 8) return k_cg_spmv_dia<8, false>;
    return k_cg_spmv_dia<16, true>;
}

int cg_dia_blocks_per_cu(int nd)
{
    static int cache[3] = {};
    int& c = cache[nd <= 5 ? 0 : (nd <= 8 ? 1 : 2)];
    if (c > 0) return c;
    int a = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, dia_kernel(nd), kBlock, 0) != hipSuccess || a < 1) a = 1;
    c = a;
    return c;
}

hipError_t launch_dia_codes(const int32_t* rp, const int32_t* col, int64_t n, int32_t S, uint32_t* out,
                            hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_dia_codes, dim3(grid_for(n, kBlock, 4096)), dim3(kBlock), 0, s, rp, col, n, S, out);
    return hipGetLastError();
}

hipError_t launch_dia_mask(const int32_t* rp, const int32_t* col, int64_t n, int32_t S, const DiaMap& m, void* mask,
                           bool m16, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const dim3 g(grid_for(n, kBlock, 4096)), blk(kBlock);
    if (m16) hipLaunchKernelGGL(k_dia_mask<uint16_t>, g, blk, 0, s, rp, col, n, S, m, static_cast<uint16_t*>(mask));
    else hipLaunchKernelGGL(k_dia_mask<uint8_t>, g, blk, 0, s, rp, col, n, S, m, static_cast<uint8_t*>(mask));
    return hipGetLastError();
}

hipError_t launch_dia_vals(const int32_t* rp, const int32_t* col, const double* vals, int64_t n, int64_t nnz, int32_t S,
                           const DiaMap& m, int nd, int batch, double* out, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    SLA_LAUNCH(k_dia_vals, dim3(grid_for(n, kBlock, 4096), batch), dim3(kBlock), 0, s, rp, col, vals, n, nnz, S, m,
               nd, out);
    return hipGetLastError();
}

hipError_t launch_cg_spmv(const CgArgs& a, int64_t k, int rp_bits, int cap, hipStream_t s)
{
    if (a.band_stride > 0 && a.dia_nd > 0)
        SLA_LAUNCH(dia_kernel(a.dia_nd), dim3(a.G, a.batch), dim3(kBlock), 0, s, a, k);
    else if (a.band_stride > 0)
        SLA_LAUNCH(band_kernel(cap, a.col16 != nullptr), dim3(a.G, a.batch), dim3(kBlock), 0, s, a, k);
    else
        SLA_LAUNCH(spmv_kernel(rp_bits, cap, off32_ok(a.n), a.split != 0, a.col16 != nullptr), dim3(a.G, a.batch),
                   dim3(kBlock), 0, s, a, k);
    return hipGetLastError();
}

hipError_t launch_cg_pupd(const CgArgs& a, int64_t k, hipStream_t s)
{
    SLA_LAUNCH(k_cg_pupd, dim3(a.Gu, a.batch), dim3(kBlock), 0, s, a, k);
    return hipGetLastError();
}

hipError_t launch_group_vals(const double* vals, double* out, int64_t nnz, int groups, const int32_t* eperm,
                             hipStream_t s)
{
    SLA_LAUNCH(k_group_vals, dim3(grid_for(nnz * kGroup, kBlock, 2048), groups), dim3(kBlock), 0, s, vals, out, nnz,
               groups, eperm);
    return hipGetLastError();
}

hipError_t launch_gcg(int which, const CgArgs& a, int64_t k, hipStream_t s)
{
    const dim3 gu(a.Gu, a.groups), gs(a.G, a.groups), blk(kBlock);
    switch (which) {
    case 0: SLA_LAUNCH(k_gcg_init, gu, blk, 0, s, a); break;
    case 1: SLA_LAUNCH(k_gcg_pupd, gu, blk, 0, s, a, k); break;
    case 2:
        if (a.g_halo > 0) {
            if (a.cap <= kGCapSmall) SLA_LAUNCH((k_gcg_spmv<kGCapSmall, true>), gs, blk, 0, s, a, k);
            else SLA_LAUNCH((k_gcg_spmv<kGCapLarge, true>), gs, blk, 0, s, a, k);
        } else {
            if (a.cap <= kGCapSmall) SLA_LAUNCH((k_gcg_spmv<kGCapSmall, false>), gs, blk, 0, s, a, k);
            else SLA_LAUNCH((k_gcg_spmv<kGCapLarge, false>), gs, blk, 0, s, a, k);
        }
        break;
    case 3: SLA_LAUNCH(k_gcg_update, gu, blk, 0, s, a, k); break;
    case 5: SLA_LAUNCH(k_gcg_diag, gu, blk, 0, s, a); break;
    default: SLA_LAUNCH(k_gcg_finish, gu, blk, 0, s, a); break;
    }
    return hipGetLastError();
}

int bs_blocks_per_cu(int rp_bits, int cap, int64_t n)
{
    static int cache[2][4][2] = {};
    const int ri = rp_bits == 64 ? 1 : 0;
    const int ci = cap <= kCapSmall ? 0 : (cap <= kCapMid ? 1 : (cap == kCapSkew ? 3 : 2));
    const bool o = off32_ok(n);
    int& c = cache[ri][ci][o ? 1 : 0];
    if (c > 0) return c;
    int a = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, spmv_kernel_mode<kSpmvBsT>(rp_bits, cap, o), kBlock, 0) !=
            hipSuccess ||
        a < 1)
        a = 1;
    c = a;
    return c;
}

hipError_t launch_bs(int which, const CgArgs& a, int64_t k, int rp_bits, int cap, hipStream_t s)
{
    const dim3 gu(a.Gu, a.batch), gs(a.G, a.batch), blk(kBlock);
    const bool o = off32_ok(a.n);
    switch (which) {
    case 0: SLA_LAUNCH(k_bs_init, gu, blk, 0, s, a); break;
    case 1: SLA_LAUNCH(k_bs_pupd, gu, blk, 0, s, a, k); break;
    case 2: SLA_LAUNCH(spmv_kernel_mode<kSpmvBsV>(rp_bits, cap, o, a.col16 != nullptr), gs, blk, 0, s, a, k); break;
    case 3: SLA_LAUNCH(k_bs_s, gu, blk, 0, s, a, k); break;
    case 4: SLA_LAUNCH(spmv_kernel_mode<kSpmvBsT>(rp_bits, cap, o, a.col16 != nullptr), gs, blk, 0, s, a, k); break;
    default: SLA_LAUNCH(k_bs_update, gu, blk, 0, s, a, k); break;
    }
    return hipGetLastError();
}

int lz_restart_rows(int64_t m)
{
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(64, kLzStage / m)));
}

hipError_t launch_lz_restart(const LzArgs& a, int64_t m, int64_t lk, hipStream_t s)
{
    if (m < 1 || m > kLzStage || lk < 1 || lk >= m) return hipErrorInvalidValue;
    const int rows = lz_restart_rows(m);
    const dim3 grid(static_cast<unsigned>((a.n + rows - 1) / rows));
    const size_t lds = sizeof(double) * static_cast<size_t>(m) * rows;
    SLA_LAUNCH(k_lz_restart, grid, dim3(kBlock), lds, s, a, m, lk, rows);
    return hipGetLastError();
}

hipError_t launch_blk_spmm(const void* rp, int rp_bits, const int32_t* col, const double* vals, const double* in,
                           const int32_t* idx_in, double* out, const int32_t* idx_out, int q, int64_t n,
                           hipStream_t s)
{
    if (q < 1 || q > kBlkMaxCols || n < 1) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>((n + kBlock - 1) / kBlock, 4096))), blk(kBlock);
    if (rp_bits == 64)
        SLA_LAUNCH((k_blk_spmm<int64_t, 8>), grid, blk, 0, s, static_cast<const int64_t*>(rp), col, vals, in, idx_in,
                   out, idx_out, q, n);
    else
        SLA_LAUNCH((k_blk_spmm<int32_t, 8>), grid, blk, 0, s, static_cast<const int32_t*>(rp), col, vals, in, idx_in,
                   out, idx_out, q, n);
    return hipGetLastError();
}

int blk_gram_groups(int64_t n)
{
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kBlkGramGroups, (n + 31) / 32)));
}

// The Gram partials part[G][mu mv] of launch_blk_gram (G returned), no reduction.
static hipError_t blk_gram_partials(const double* A, const int32_t* ia, int mu, const double* B, const int32_t* ib,
                                    int mv, int64_t n, double* part, hipStream_t s, bool same, int* Gout);

hipError_t launch_blk_gram(const double* A, const int32_t* ia, int mu, const double* B, const int32_t* ib, int mv,
                           int64_t n, double* part, double* out, hipStream_t s, bool same, double* yproj)
{
    if ((same && mu != mv) || (yproj && mu < mv)) return hipErrorInvalidValue;
    int G = 0;
    hipError_t e = blk_gram_partials(A, ia, mu, B, ib, mv, n, part, s, same, &G);
    if (e != hipSuccess) return e;
    const int np = mu * mv;
    SLA_LAUNCH(k_blk_reduce, dim3(static_cast<unsigned>(np)), dim3(kBlock), 0, s, part, G, np, out, yproj, mv);
    return hipGetLastError();
}

hipError_t launch_blk_gram_orth(const double* A, const int32_t* ia, int w, int64_t n, double* part, double* gram,
                                bool scale, double pivot, double* flag, double* T, hipStream_t s)
{
    if (w < 1 || w > kCoefMax) return hipErrorInvalidValue;
    hipError_t e = launch_blk_gram(A, ia, w, A, ia, w, n, part, gram, s, true);
    if (e != hipSuccess) return e;
    SLA_LAUNCH(k_blk_orth_coef, dim3(1), dim3(64), 0, s, gram, w, scale ? 1 : 0, pivot, flag, T);
    return hipGetLastError();
}

static hipError_t blk_gram_partials(const double* A, const int32_t* ia, int mu, const double* B, const int32_t* ib,
                                    int mv, int64_t n, double* part, hipStream_t s, bool same, int* Gout)
{
    if (mu < 1 || mv < 1 || mu > kBlkMaxCols || mv > kBlkMaxCols || n < 1) return hipErrorInvalidValue;
    if (same && mu != mv) return hipErrorInvalidValue;
    const int np = mu * mv;
    const bool pieces = n % 2 == 0 && !(reinterpret_cast<uintptr_t>(A) & 15) && !(reinterpret_cast<uintptr_t>(B) & 15);
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
        ncu = 1;
    if (pieces) {
        // at most 8 register tiles of 4 x 4 (1 wide where a side is narrower than 4): the
        // products stream from registers like the combinations
        const int TA = mu >= 4 ? 4 : 1, TB = mv >= 4 ? 4 : 1;
        const int ntile = ((mu + TA - 1) / TA) * ((mv + TB - 1) / TB);
        int ntp = 1;
        while (ntp < ntile) ntp *= 2;
        // wider blocks of at most 24 x 24 columns: 6 x 6 tiles, at most 16
        const bool wide = ntp > 8 && mu <= 24 && mv <= 24;
        if (wide) ntp = ((mu + 5) / 6) * ((mv + 5) / 6) <= 4 ? 4 : 16;
        if (ntp <= 8 || wide) {
            const double* Bs = same ? A : B;
            const int32_t* ibs = same ? ia : ib;
            using RtKernel = void (*)(const double*, const int32_t*, int, const double*, const int32_t*, int, int64_t,
                                      double*);
            RtKernel f = nullptr;
#define SLA_GRAM_RT(ta, tb)                                                                                \
    f = ntp == 1 ? k_blk_gram_rt<ta, tb, 1> : ntp == 2 ? k_blk_gram_rt<ta, tb, 2>                         \
        : ntp == 4 ? k_blk_gram_rt<ta, tb, 4> : k_blk_gram_rt<ta, tb, 8>
            if (wide) f = ntp == 4 ? k_blk_gram_rt<6, 6, 4> : k_blk_gram_rt<6, 6, 16>;
            else if (TA == 1 && TB == 1) SLA_GRAM_RT(1, 1);
            else if (TA == 4 && TB == 1) SLA_GRAM_RT(4, 1);
            else if (TA == 1) SLA_GRAM_RT(1, 4);
            else SLA_GRAM_RT(4, 4);
#undef SLA_GRAM_RT
            int occ = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, f, kBlock, 0) != hipSuccess || occ < 1) occ = 1;
            const int64_t per_block = (kBlock / 64) * (64 / ntp);   // row pairs per grid step of a workgroup
            const int G = static_cast<int>(std::min<int64_t>(
                {static_cast<int64_t>(blk_gram_groups(n)), (n / 2 + per_block - 1) / per_block,
                 static_cast<int64_t>(occ) * ncu}));
            SLA_LAUNCH(f, dim3(static_cast<unsigned>(G)), dim3(kBlock), 0, s, A, ia, mu, Bs, ibs, mv, n, part);
            *Gout = G;
            return hipGetLastError();
        }
    }
    if (pieces) {
        // pipelined slices of 16-byte pieces: ncol R <= 4096 doubles (32 KiB of LDS)
        const int ncol = same ? mu : mu + mv;
        int R = 4096;
        while (ncol * R > 4096) R /= 2;
        int lgh = 0;
        while ((2 << lgh) < R) ++lgh;
        const int64_t nslices = (n + R - 1) / R;
        const size_t lds = sizeof(double) * std::max<size_t>(static_cast<size_t>(ncol) * (R + 2), kBlock);
        const int TA = mu >= 4 ? 4 : 1, TB = mv >= 4 ? 4 : 1;
        const int ntile = ((mu + TA - 1) / TA) * ((mv + TB - 1) / TB);
        int tpt = 1;   // threads per tile: a power of 2 with ntile tpt <= kBlock
        while (ntile * tpt * 2 <= kBlock) tpt *= 2;
        const int pt = (ntile + kBlock / tpt - 1) / (kBlock / tpt);
        const int sm = same ? 1 : 0;
        using GramKernel = void (*)(const double*, const int32_t*, int, const double*, const int32_t*, int, int,
                                    int64_t, int, int, double*);
        GramKernel f = (TA == 1 && TB == 1) ? k_blk_gram_pipe<1, 1, 1, 8>
                       : (TA == 4 && TB == 1) ? k_blk_gram_pipe<4, 1, 1, 8>
                       : (TA == 1)           ? k_blk_gram_pipe<1, 4, 1, 8>
                       : (pt <= 1)           ? k_blk_gram_pipe<4, 4, 1, 8>
                       : (pt <= 2)           ? k_blk_gram_pipe<4, 4, 2, 8>
                                             : k_blk_gram_pipe<4, 4, 3, 8>;
        // one resident round of workgroups (a second, partial round would run on part of
        // the GPU), each taking slices grid-stride
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, f, kBlock, lds) != hipSuccess || occ < 1) occ = 1;
        const int G = static_cast<int>(std::min<int64_t>({static_cast<int64_t>(blk_gram_groups(n)), nslices,
                                                          static_cast<int64_t>(occ) * ncu}));
        const dim3 grid(static_cast<unsigned>(G)), blk(kBlock);
        SLA_LAUNCH(f, grid, blk, lds, s, A, ia, mu, B, ib, mv, sm, n, lgh, tpt, part);
        *Gout = G;
        return hipGetLastError();
    }
    if (same) B = A, ib = ia;
    // slice rows: (mu + mv) (R + 1) doubles within 32 KiB of LDS (five workgroups per
    // CU keep loads in flight while others compute), R a multiple of 32
    constexpr int kStage = 4000;
    const int R = std::max(32, std::min(1024, (kStage / (mu + mv) - 1) / 32 * 32));
    const int64_t nslices = (n + R - 1) / R;
    const int G = static_cast<int>(std::min<int64_t>(blk_gram_groups(n), nslices));
    // the LDS holds the staged slice and, at the end, kBlock partial sums
    const size_t lds = sizeof(double) * std::max<size_t>(static_cast<size_t>(mu + mv) * (R + 1), kBlock);
    const dim3 grid(static_cast<unsigned>(G)), blk(kBlock);
    if (np > kBlock) {   // many pairs: 4 x 4 register tiles
        const int ntile = ((mu + 3) / 4) * ((mv + 3) / 4);
        int tpt = 1;   // threads per tile: a power of 2 with ntile tpt <= kBlock
        while (ntile * tpt * 2 <= kBlock) tpt *= 2;
        const int pt = (ntile + kBlock / tpt - 1) / (kBlock / tpt);
        if (pt <= 1) SLA_LAUNCH(k_blk_gram_tiled<1>, grid, blk, lds, s, A, ia, mu, B, ib, mv, n, R, tpt, part);
        else if (pt <= 2) SLA_LAUNCH(k_blk_gram_tiled<2>, grid, blk, lds, s, A, ia, mu, B, ib, mv, n, R, tpt, part);
        else SLA_LAUNCH(k_blk_gram_tiled<3>, grid, blk, lds, s, A, ia, mu, B, ib, mv, n, R, tpt, part);
        *Gout = G;
        return hipGetLastError();
    }
    int tpp = 1;   // threads per pair: a power of 2 with np tpp <= kBlock
    while (np * tpp * 2 <= kBlock) tpp *= 2;
    const int pp = (np + kBlock - 1) / kBlock;
    if (pp <= 1) SLA_LAUNCH(k_blk_gram<1>, grid, blk, lds, s, A, ia, mu, B, ib, mv, n, R, tpp, part);
    else if (pp <= 2) SLA_LAUNCH(k_blk_gram<2>, grid, blk, lds, s, A, ia, mu, B, ib, mv, n, R, 1, part);
    else if (pp <= 4) SLA_LAUNCH(k_blk_gram<4>, grid, blk, lds, s, A, ia, mu, B, ib, mv, n, R, 1, part);
    else if (pp <= 8) SLA_LAUNCH(k_blk_gram<8>, grid, blk, lds, s, A, ia, mu, B, ib, mv, n, R, 1, part);
    else if (pp <= 16) SLA_LAUNCH(k_blk_gram<16>, grid, blk, lds, s, A, ia, mu, B, ib, mv, n, R, 1, part);
    else SLA_LAUNCH(k_blk_gram<(kBlkMaxCols * kBlkMaxCols + kBlock - 1) / kBlock>, grid, blk, lds, s, A, ia, mu, B,
                    ib, mv, n, R, 1, part);
    *Gout = G;
    return hipGetLastError();
}

hipError_t launch_blk_reduce(const double* part, int G, int np, double* out, hipStream_t s)
{
    if (G < 1 || np < 1) return hipErrorInvalidValue;
    SLA_LAUNCH(k_blk_reduce, dim3(static_cast<unsigned>(np)), dim3(kBlock), 0, s, part, G, np, out, nullptr, 0);
    return hipGetLastError();
}

hipError_t launch_blk_diag_inv(const void* rp, int rp_bits, const int32_t* col, const double* vals, int64_t n,
                               double* tinv, double* part, hipStream_t s)
{
    const dim3 grid(static_cast<unsigned>(blk_comb_groups(n))), blk(kBlock);
    if (rp_bits == 64)
        SLA_LAUNCH(k_blk_diag_inv<int64_t>, grid, blk, 0, s, static_cast<const int64_t*>(rp), col, vals, n, tinv, part);
    else
        SLA_LAUNCH(k_blk_diag_inv<int32_t>, grid, blk, 0, s, static_cast<const int32_t*>(rp), col, vals, n, tinv, part);
    return hipGetLastError();
}

hipError_t launch_blk_comb_dual(const double* in, const int32_t* idx_in, int m, int j0, const double* Y,
                                double* out, const int32_t* idx_out, const int32_t* idx_out2, int q, int64_t n,
                                hipStream_t s)
{
    if (m < 1 || j0 < 0 || j0 >= m || q < 1 || q > 32 || n < 1) return hipErrorInvalidValue;
    if ((n & 1) || (reinterpret_cast<uintptr_t>(in) & 15) || (reinterpret_cast<uintptr_t>(out) & 15))
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blk_comb_groups(n))), blk(kBlock);
    if (q <= 1) SLA_LAUNCH(k_blk_comb2d<1>, grid, blk, 0, s, in, idx_in, m, j0, Y, out, idx_out, idx_out2, q, n);
    else if (q <= 2) SLA_LAUNCH(k_blk_comb2d<2>, grid, blk, 0, s, in, idx_in, m, j0, Y, out, idx_out, idx_out2, q, n);
    else if (q <= 4) SLA_LAUNCH(k_blk_comb2d<4>, grid, blk, 0, s, in, idx_in, m, j0, Y, out, idx_out, idx_out2, q, n);
    else if (q <= 8) SLA_LAUNCH(k_blk_comb2d<8>, grid, blk, 0, s, in, idx_in, m, j0, Y, out, idx_out, idx_out2, q, n);
    else if (q <= 16) SLA_LAUNCH(k_blk_comb2d<16>, grid, blk, 0, s, in, idx_in, m, j0, Y, out, idx_out, idx_out2, q, n);
    else SLA_LAUNCH(k_blk_comb2d<32>, grid, blk, 0, s, in, idx_in, m, j0, Y, out, idx_out, idx_out2, q, n);
    return hipGetLastError();
}

hipError_t launch_blk_rowscale(const double* in, const int32_t* idx_in, double* out, const int32_t* idx_out, int q,
                               int64_t n, const double* t, hipStream_t s)
{
    if (q < 1 || n < 1) return hipErrorInvalidValue;
    SLA_LAUNCH(k_blk_rowscale, dim3(static_cast<unsigned>(blk_comb_groups(n))), dim3(kBlock), 0, s, in, idx_in, out,
               idx_out, q, n, t);
    return hipGetLastError();
}

int blk_comb_groups(int64_t n)
{
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(1024, (n + kBlock - 1) / kBlock)));
}

hipError_t launch_blk_comb(const double* in, const int32_t* idx_in, int m, const double* Y, double* out,
                           const int32_t* idx_out, int q, int64_t n, double* part, hipStream_t s, bool pairs)
{
    if (m < 1 || q < 1 || q > 32 || n < 1) return hipErrorInvalidValue;
    if (pairs && ((n & 1) || (reinterpret_cast<uintptr_t>(in) & 15) || (reinterpret_cast<uintptr_t>(out) & 15)))
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blk_comb_groups(n))), blk(kBlock);
    if (pairs) {
        if (q <= 1) SLA_LAUNCH(k_blk_comb2<1>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
        else if (q <= 2) SLA_LAUNCH(k_blk_comb2<2>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
        else if (q <= 4) SLA_LAUNCH(k_blk_comb2<4>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
        else if (q <= 8) SLA_LAUNCH(k_blk_comb2<8>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
        else if (q <= 16) SLA_LAUNCH(k_blk_comb2<16>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
        else SLA_LAUNCH(k_blk_comb2<32>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
        return hipGetLastError();
    }
    if (q <= 1) SLA_LAUNCH(k_blk_comb<1>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
    else if (q <= 2) SLA_LAUNCH(k_blk_comb<2>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
    else if (q <= 4) SLA_LAUNCH(k_blk_comb<4>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
    else if (q <= 8) SLA_LAUNCH(k_blk_comb<8>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
    else if (q <= 16) SLA_LAUNCH(k_blk_comb<16>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
    else SLA_LAUNCH(k_blk_comb<32>, grid, blk, 0, s, in, idx_in, m, Y, out, idx_out, q, n, part);
    return hipGetLastError();
}

hipError_t launch_lz_axpy_dots(const LzArgs& a, int64_t ncols, hipStream_t s)
{
    if (ncols < 1 || ncols > kLzFusedCols) return hipErrorInvalidValue;
    static_assert(kBlock / 64 == 4 && kLzRows % kBlock == 0, "four waves, whole trips");
    SLA_LAUNCH(k_lz_axpy_dots<kLzFusedCols>, dim3(static_cast<unsigned>(a.Gd)), dim3(kBlock), 0, s, a,
               static_cast<int>(ncols));
    return hipGetLastError();
}

hipError_t launch_lz(int which, const LzArgs& a, int64_t j, double nrm, int last, hipStream_t s)
{
    const dim3 gu(a.Gu), blk(kBlock);
    switch (which) {
    case 0: SLA_LAUNCH(k_lz_norm, gu, blk, 0, s, a); break;
    case 1: SLA_LAUNCH(k_lz_start, gu, blk, 0, s, a, nrm); break;
    case 2: SLA_LAUNCH(k_lz_three, gu, blk, 0, s, a, j); break;
    case 3: SLA_LAUNCH(k_lz_dots, dim3(a.Gd), blk, 0, s, a, j); break;
    case 4: SLA_LAUNCH(k_lz_reduce, dim3(static_cast<unsigned>(std::min<int64_t>(j, 1024))), blk, 0, s, a, j);
        break;
    case 5: SLA_LAUNCH(k_lz_axpy, gu, blk, 0, s, a, j, last); break;
    case 6: SLA_LAUNCH(k_lz_next, gu, blk, 0, s, a, j); break;
    case 7:
        if (a.k <= 1) SLA_LAUNCH(k_lz_ritz<1>, gu, blk, 0, s, a);
        else if (a.k <= 2) SLA_LAUNCH(k_lz_ritz<2>, gu, blk, 0, s, a);
        else if (a.k <= 4) SLA_LAUNCH(k_lz_ritz<4>, gu, blk, 0, s, a);
        else if (a.k <= 8) SLA_LAUNCH(k_lz_ritz<8>, gu, blk, 0, s, a);
        else if (a.k <= 16) SLA_LAUNCH(k_lz_ritz<16>, gu, blk, 0, s, a);
        else SLA_LAUNCH(k_lz_ritz<kEigMaxK>, gu, blk, 0, s, a);
        break;
    default: SLA_LAUNCH(k_lz_scale, gu, blk, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_eig_grad(const void* row_ptr, int rp_bits, const int32_t* col, const double* U, const double* g,
                           int k, int64_t n, int64_t nnz, double* gvals, hipStream_t s)
{
    if (n == 0 || nnz == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((n + kTile - 1) / kTile)), blk(kBlock);
    if (rp_bits == 64)
        SLA_LAUNCH(k_eig_grad<int64_t>, grid, blk, 0, s, static_cast<const int64_t*>(row_ptr), col, U, g, k, n,
                   gvals);
    else
        SLA_LAUNCH(k_eig_grad<int32_t>, grid, blk, 0, s, static_cast<const int32_t*>(row_ptr), col, U, g, k, n,
                   gvals);
    return hipGetLastError();
}

hipError_t launch_pack_pattern(const void* rp, int rp_bits, const int32_t* col, int64_t n, int64_t nnz, int64_t r0,
                               int64_t e0, int64_t rows_padded, void* out_rp, int out_bits, int32_t* out_col,
                               hipStream_t s)
{
    const dim3 grid(grid_for(std::max(rows_padded + 1, nnz), kBlock, 4096)), blk(kBlock);
    if (rp_bits == 64 && out_bits == 64)
        SLA_LAUNCH((k_pack_pattern<int64_t, int64_t>), grid, blk, 0, s, static_cast<const int64_t*>(rp), col, n, nnz,
                   r0, e0, rows_padded, static_cast<int64_t*>(out_rp), out_col);
    else if (rp_bits == 64)
        SLA_LAUNCH((k_pack_pattern<int64_t, int32_t>), grid, blk, 0, s, static_cast<const int64_t*>(rp), col, n, nnz,
                   r0, e0, rows_padded, static_cast<int32_t*>(out_rp), out_col);
    else if (out_bits == 64)
        SLA_LAUNCH((k_pack_pattern<int32_t, int64_t>), grid, blk, 0, s, static_cast<const int32_t*>(rp), col, n, nnz,
                   r0, e0, rows_padded, static_cast<int64_t*>(out_rp), out_col);
    else
        SLA_LAUNCH((k_pack_pattern<int32_t, int32_t>), grid, blk, 0, s, static_cast<const int32_t*>(rp), col, n, nnz,
                   r0, e0, rows_padded, static_cast<int32_t*>(out_rp), out_col);
    return hipGetLastError();
}

hipError_t launch_cg_update(const CgArgs& a, int64_t k, hipStream_t s)
{
    const dim3 grid(a.Gu, a.batch), blk(kBlock);
    if (a.wide_update) {
        if (a.jacobi) {
            if (a.stream_nt) SLA_LAUNCH((k_cg_update_wide<true, true>), grid, blk, 0, s, a, k);
            else SLA_LAUNCH((k_cg_update_wide<false, true>), grid, blk, 0, s, a, k);
        } else {
            if (a.stream_nt) SLA_LAUNCH((k_cg_update_wide<true, false>), grid, blk, 0, s, a, k);
            else SLA_LAUNCH((k_cg_update_wide<false, false>), grid, blk, 0, s, a, k);
        }
        return hipGetLastError();
    }
    if (a.jacobi) {
        if (a.stream_nt) SLA_LAUNCH((k_cg_update<true, true>), grid, blk, 0, s, a, k);
        else SLA_LAUNCH((k_cg_update<false, true>), grid, blk, 0, s, a, k);
    } else {
        if (a.stream_nt) SLA_LAUNCH((k_cg_update<true, false>), grid, blk, 0, s, a, k);
        else SLA_LAUNCH((k_cg_update<false, false>), grid, blk, 0, s, a, k);
    }
    return hipGetLastError();
}

hipError_t launch_matvec(const void* row_ptr, int rp_bits, const int32_t* col, const double* vals,
                         const double* x, double* y, int64_t n_rows, int64_t nnz, int64_t n_cols, int batch,
                         int cap, hipStream_t s)
{
    if (n_rows == 0) return hipSuccess;
    if (rp_bits == 64)
        return launch_matvec_any(static_cast<const int64_t*>(row_ptr), col, vals, x, y, n_rows, nnz, n_cols, batch,
                                 cap, s);
    return launch_matvec_any(static_cast<const int32_t*>(row_ptr), col, vals, x, y, n_rows, nnz, n_cols, batch,
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
        SLA_LAUNCH(k_pattern_outer<int64_t>, grid, block, 0, s, static_cast<const int64_t*>(row_ptr), col,
                           sign, u, us, v, vs, g, n_rows, nnz);
    else
        SLA_LAUNCH(k_pattern_outer<int32_t>, grid, block, 0, s, static_cast<const int32_t*>(row_ptr), col,
                           sign, u, us, v, vs, g, n_rows, nnz);
    return hipGetLastError();
}

hipError_t launch_gather_vals(const int64_t* perm, const double* vals, double* out, int64_t nnz, int batch,
                              hipStream_t s)
{
    if (nnz == 0) return hipSuccess;
    SLA_LAUNCH(k_gather_vals, dim3(grid_for(nnz, kBlock, 4096), batch), dim3(kBlock), 0, s, perm, vals,
                       out, nnz);
    return hipGetLastError();
}

hipError_t launch_validate(const void* row_ptr, int rp_bits, const int32_t* col, int64_t n_rows, int64_t n_cols,
                           int64_t nnz, int32_t* out, hipStream_t s)
{
    const int64_t ntiles = (n_rows + kTile - 1) / kTile;
    const dim3 grid(static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(ntiles, 8192)))), block(kBlock);
    if (rp_bits == 64)
        hipLaunchKernelGGL(k_validate<int64_t>, grid, block, 0, s, static_cast<const int64_t*>(row_ptr), col, n_rows,
                           n_cols, nnz, out);
    else
        hipLaunchKernelGGL(k_validate<int32_t>, grid, block, 0, s, static_cast<const int32_t*>(row_ptr), col, n_rows,
                           n_cols, nnz, out);
    return hipGetLastError();
}

hipError_t launch_narrow_rp(const int64_t* in, int32_t* out, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(k_narrow_i32, dim3(grid_for(n, kBlock, 8192)), dim3(kBlock), 0, s, in, out, n);
    return hipGetLastError();
}

hipError_t launch_colb16(const int32_t* rp, const int32_t* col, int16_t* out, int64_t n_rows, int32_t S,
                         hipStream_t s)
{
    hipLaunchKernelGGL(k_colb16, dim3(grid_for(n_rows, kBlock, 8192)), dim3(kBlock), 0, s, rp, col, out, n_rows, S);
    return hipGetLastError();
}

hipError_t launch_col16(const int32_t* rp, const int32_t* col, int16_t* out, int64_t n_rows, hipStream_t s)
{
    const int64_t ntiles = (n_rows + kTile - 1) / kTile;
    hipLaunchKernelGGL(k_col16, dim3(grid_for(ntiles, 1, 8192)), dim3(kBlock), 0, s, rp, col, out, n_rows);
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
