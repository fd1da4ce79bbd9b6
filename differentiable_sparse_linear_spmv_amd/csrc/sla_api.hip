// sla_api.hip -- the C ABI declared in include/sla.h: handles, argument checks,
// workspace, and the host drivers that enqueue the CG and adjoint kernels.
//
// The solve loop follows the conjugate-gradient method of torch-sla's
// pytorch-native backend (paperpeel page, sections 1 and 3.1), driven from the
// device: the host enqueues chunks of iterations without reading any scalar, and
// polls a device counter of still-running systems once per chunk (two chunks are
// kept in flight, so the GPU never waits on the host).  The backward pass is the
// linear adjoint of the gist.science summaries (Methodology item 2): a second CG
// on A^T (A itself when the caller declares it symmetric), then an O(nnz) outer
// product on the pattern (paperpeel section 3.2.3).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <map>
#include <unordered_map>
#include <vector>

#include "sla.h"
#include "sla_internal.h"

using namespace sla;

struct sla_csr {
    int64_t n_rows = 0, n_cols = 0, nnz = 0;
    int32_t rp_bits = 32;
    uint32_t flags = 0;
    const void* row_ptr = nullptr;
    const int32_t* col = nullptr;
    // Row pointers the kernels read: the caller's, or an owned 32-bit copy of 64-bit
    // row pointers when nnz < 2^31 (4 bytes per row less traffic in every SpMV).
    const void* krp = nullptr;
    int32_t krp_bits = 32;
    void* rp_owned = nullptr;
    // 16-bit column offsets (column minus the first row of its 256-row tile) that the
    // staged CG / BiCGStab SpMV reads instead of the 32-bit columns: 2 bytes per entry
    // less in every product.  Built at create when every |c - i| <= kCol16MaxSpan
    // (SLA_COL16=0 turns them off); null otherwise.
    // A banded handle builds them on first use only (its CG SpMV reads colb16 instead).
    int16_t* col16 = nullptr;
    bool c16_ok = false;          // every |c - i| <= kCol16MaxSpan: col16 may be built
    int16_t* col16_t = nullptr;   // the same for the transposed pattern
    int16_t* colb16 = nullptr;    // banded pattern: offsets from the first row of the
                                  // line-walking SpMV's window of each row
    int device = 0;
    int n_cu = 256;
    int cap = kCapSmall;        // LDS variant for A
    int32_t tile_max = 0;
    int32_t row_max = 0;
    // Banded pattern (line-walking SpMV): line stride S, 0 if the plain SpMV is used.
    int64_t band = 0;
    int band_cap = kCapSmall;
    // Diagonal layout of a banded pattern with at most kDiaMax distinct offsets (the CG
    // SpMV k_cg_spmv_dia): dia_nd diagonals (0: none), their codes' map, per-row masks
    // (uint8, or uint16 above 8 diagonals), and the values in that layout [batch][nd][n],
    // rewritten by each solve (SLA_DIA=0 at create turns the layout off).
    int dia_nd = 0;
    bool dia_align = true;   // line stride = 8 (mod 16): windows shifted onto 128-byte boundaries (SLA_DIA_ALIGN=0: not)
    DiaMap dia_map{};
    int8_t dia_b[kDiaMax] = {};
    int8_t dia_e[kDiaMax] = {};
    void* dia_mask = nullptr;
    double* dia_vals = nullptr;
    size_t dia_vals_bytes = 0;
    // Split CG schedule (unstructured patterns); the transposed pattern has the same span.
    bool split = false;
    // Grouped kernels for batches of split-schedule patterns (SLA_CG_GROUPED=0 turns them off).
    bool group_ok = true;
    // The grouped kernels run on a reverse Cuthill-McKee reordering of the pattern, built on
    // the first grouped solve (SLA_CG_REORDER=0 turns it off): row pointers, columns, the
    // entry permutation and the row permutation (new -> caller's), all int32.
    bool reorder_ok = true;
    bool g_win_ok = true;   // the grouped SpMV may keep its operand in an LDS window (SLA_GCG_WINDOW=0: never)
    bool g_reordered = false;
    int32_t *g_rp = nullptr, *g_col = nullptr, *g_eperm = nullptr, *g_perm = nullptr;
    int16_t* g_col16 = nullptr;   // reordered columns minus the first row of their 64-row tile (g_halo > 0)
    int32_t g_halo = 0;   // operand window of the grouped SpMV on the reordered pattern (0: none)
    // transposed pattern (lazily built unless SLA_SYMMETRIC)
    bool has_t = false;
    void* row_ptr_t = nullptr;
    int32_t* col_t = nullptr;
    int64_t* perm_t = nullptr;
    int cap_t = kCapSmall;
    // workspace
    void* ws = nullptr;
    size_t ws_bytes = 0;
    double* vals_t = nullptr;   // [batch][nnz] transposed values
    // grouped batches: x and the values in the grouped layout
    void* gws = nullptr;
    size_t gws_bytes = 0;
    size_t vals_t_bytes = 0;
    int32_t* flag_host = nullptr;   // pinned, 2 slots for the polling copies
    // Lanczos (sla_eigsh): device workspace and a pinned host staging area
    void* eig_ws = nullptr;
    size_t eig_ws_bytes = 0;
    double* eig_host = nullptr;
    size_t eig_host_bytes = 0;
    // LOBPCG (sla_lobpcg): block vectors and scratch on the device, a pinned arena
    void* lob_ws = nullptr;
    size_t lob_ws_bytes = 0;
    char* lob_host = nullptr;
    size_t lob_host_bytes = 0;
    double* lob_res = nullptr;   // coherent pinned memory the kernels write results into
    size_t lob_res_bytes = 0;
    hipEvent_t poll_ev[2] = {nullptr, nullptr};
    std::mutex mu;
};

// SparseTensorList: items with distinct patterns packed block-diagonally into one
// pattern, each item's rows starting on a tile boundary.
struct sla_list {
    int32_t items = 0;
    uint32_t flags = 0;
    int device = 0;
    std::vector<int64_t> n, nnz, r0, e0;   // per item: rows, entries, first packed row / entry
    int64_t n_total = 0, nnz_total = 0;
    sla_csr* packed = nullptr;             // handle of the packed pattern
    void* rp = nullptr;                    // owned packed row pointers (32- or 64-bit)
    int32_t* col = nullptr;                // owned packed columns
    int32_t* d_wg = nullptr;               // per-system tables (ListPlan)
    int64_t* d_tiles = nullptr;
    int64_t* d_rend = nullptr;
    int32_t total_wg = 0;
    double* stage = nullptr;               // packed values, three packed vectors, packed gradient
    size_t stage_bytes = 0;
    std::mutex mu;
};

namespace {

thread_local char g_err[512] = "";

sla_status fail(sla_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

#define HIP_TRY(expr)                                                                    \
    do {                                                                                 \
        hipError_t e_ = (expr);                                                          \
        if (e_ != hipSuccess)                                                            \
            return fail(SLA_ERR_HIP, "%s: %s (%s:%d)", #expr, hipGetErrorString(e_),     \
                        __FILE__, __LINE__);                                             \
    } while (0)

// ---------------------------------------------------------------- kernel timing
struct Pending {
    int kid;
    hipEvent_t a, b;
    double bytes;   // algorithmic bytes of what was timed (0 where not counted)
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
int64_t g_launches[SLA_K_COUNT] = {};
double g_ms[SLA_K_COUNT] = {};
double g_bytes[SLA_K_COUNT] = {};

hipEvent_t pool_get()
{
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Time what f() enqueues.  single: f launches exactly one kernel, whose own start
// and end are recorded (hipExtLaunchKernelGGL events); otherwise events bracket f.
template <class F>
hipError_t timed(int kid, hipStream_t s, F&& f, bool single = true, double bytes = 0.0)
{
    bool on;
    {
        std::lock_guard<std::mutex> lk(g_tmu);
        on = g_timing;
    }
    if (!on) return f();
    hipEvent_t a, b;
    {
        std::lock_guard<std::mutex> lk(g_tmu);
        a = pool_get();
        b = pool_get();
    }
    if (!a || !b) return f();
    hipError_t e;
    if (single) {
        launch_events() = LaunchEvents{a, b};
        e = f();
        launch_events() = LaunchEvents{};
    } else {
        (void)hipEventRecord(a, s);
        e = f();
        (void)hipEventRecord(b, s);
    }
    std::lock_guard<std::mutex> lk(g_tmu);
    g_pending.push_back({kid, a, b, bytes});
    return e;
}

hipError_t timing_collect()
{
    std::vector<Pending> todo;
    {
        std::lock_guard<std::mutex> lk(g_tmu);
        todo.swap(g_pending);
    }
    hipError_t first = hipSuccess;
    for (auto& p : todo) {
        hipError_t e = hipEventSynchronize(p.b);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.a, p.b);
        if (e != hipSuccess && first == hipSuccess) first = e;
        std::lock_guard<std::mutex> lk(g_tmu);
        if (e == hipSuccess) {
            g_launches[p.kid] += 1;
            g_ms[p.kid] += ms;
            g_bytes[p.kid] += p.bytes;
        }
        g_pool.push_back(p.a);
        g_pool.push_back(p.b);
    }
    return first;
}

// ---------------------------------------------------------------- helpers
sla_status check_device(const sla_csr* A)
{
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (dev != A->device)
        return fail(SLA_ERR_INVALID_ARG, "handle was created on device %d, current device is %d", A->device, dev);
    return SLA_OK;
}

// Device memory of the library: from the caller's allocator when one is registered
// (sla_set_allocator), else hipMalloc.  Every block remembers the free function that
// owns it, so a later change of allocator never frees through the wrong one.
struct AllocHook {
    sla_alloc_fn alloc = nullptr;
    sla_free_fn free = nullptr;
    void* ctx = nullptr;
};
std::mutex g_amu;
AllocHook g_hook;
std::unordered_map<void*, AllocHook> g_hooked;   // blocks from a registered allocator

sla_status dev_alloc(void** p, size_t bytes)
{
    *p = nullptr;
    if (bytes == 0) return SLA_OK;
    AllocHook h;
    {
        std::lock_guard<std::mutex> lk(g_amu);
        h = g_hook;
    }
    if (h.alloc) {
        void* q = h.alloc(bytes, nullptr, h.ctx);
        if (!q) return fail(SLA_ERR_OOM, "the registered allocator returned NULL for %zu bytes", bytes);
        std::lock_guard<std::mutex> lk(g_amu);
        g_hooked[q] = h;
        *p = q;
        return SLA_OK;
    }
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        return fail(SLA_ERR_OOM, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
    }
    return SLA_OK;
}

// Frees a block of dev_alloc.  A block of a registered allocator goes back to it after
// the device has finished with it (such allocators pool by stream, and the library may
// have used the block on any stream).
hipError_t dev_free(void* p)
{
    if (!p) return hipSuccess;
    AllocHook h;
    bool hooked = false;
    {
        std::lock_guard<std::mutex> lk(g_amu);
        auto it = g_hooked.find(p);
        if (it != g_hooked.end()) {
            h = it->second;
            hooked = true;
            g_hooked.erase(it);
        }
    }
    if (!hooked) return hipFree(p);
    hipError_t e = hipDeviceSynchronize();
    h.free(p, nullptr, h.ctx);
    return e;
}

int choose_cap(int32_t tile_max, int32_t row_max)
{
    if (row_max > kBinLaneMax) return kCapSkew;
    if (tile_max <= kCapSmall) return kCapSmall;
    if (tile_max <= kCapMid) return kCapMid;
    return kCapLarge;
}

constexpr size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Workgroups per system: the grid of the CG kernels fills every CU exactly once
// (resident workgroups per CU from the occupancy of the SpMV variant in use), so the
// grid-stride loops have no second, partial wave of workgroups.
int blocks_per_system(const sla_csr* A, int64_t ntiles, int64_t batch, int per_cu)
{
    if (batch >= 8 && batch % 8 == 0) {
        // one XCD per system: about 8 tiles per workgroup, a multiple of 8 workgroups
        int64_t g = (ntiles + 7) / 8;
        g = std::max<int64_t>(8, std::min<int64_t>(256, (g + 7) & ~int64_t(7)));
        return static_cast<int>(g);
    }
    int64_t target = static_cast<int64_t>(A->n_cu) * per_cu;
    int64_t g = (target + batch - 1) / batch;
    if (g >= 8) g &= ~int64_t(7);   // a multiple of 8 enables the XCD band mapping
    g = std::min<int64_t>(g, std::max<int64_t>(ntiles, 1));
    return static_cast<int>(std::max<int64_t>(g, 1));
}

struct Workspace {
    double *r, *p0, *p1, *q, *z, *dg, *part_sigma, *part_rho, *part_rr, *part_aux, *part_tt;
    SysState* st;
    int32_t* n_active;
};

// Solver methods and the workspace each needs.
enum Method { kMethodCG = 0, kMethodJacobi = 1, kMethodBiCGStab = 2 };
// vectors r, p0, p1, q (+ z, dg with Jacobi; + z with BiCGStab);
// partials sigma, rho (+ rr, aux with Jacobi; + rr, aux, tt with BiCGStab)
constexpr int kWsVectors[3] = {4, 6, 5};
constexpr int kWsPartials[3] = {2, 4, 5};

size_t workspace_bytes(int64_t n, int64_t batch, int G, int method, int64_t nstate)
{
    const size_t vec = align256(sizeof(double) * static_cast<size_t>(n) * batch);
    const size_t part = align256(sizeof(double) * static_cast<size_t>(G) * batch);
    return kWsVectors[method] * vec + kWsPartials[method] * part + align256(sizeof(SysState) * nstate) + 256;
}

// The workspace's arrays carved from one block at p (workspace_bytes of the same
// arguments).  nstate: the number of systems (batch, or the items of a
// SparseTensorList; < 0: batch).
void carve_workspace(char* p, int64_t n, int64_t batch, int G, Workspace* w, int method, int64_t nstate)
{
    if (nstate < 0) nstate = batch;
    const size_t vec = align256(sizeof(double) * static_cast<size_t>(n) * batch);
    const size_t part = align256(sizeof(double) * static_cast<size_t>(G) * batch);
    const int nv = kWsVectors[method], np = kWsPartials[method];
    auto vec_at = [&](int i) { return i < nv ? reinterpret_cast<double*>(p + i * vec) : nullptr; };
    auto part_at = [&](int i) { return i < np ? reinterpret_cast<double*>(p + nv * vec + i * part) : nullptr; };
    w->r = vec_at(0);
    w->p0 = vec_at(1);
    w->p1 = vec_at(2);
    w->q = vec_at(3);
    w->z = vec_at(4);
    w->dg = vec_at(5);
    w->part_sigma = part_at(0);
    w->part_rho = part_at(1);
    w->part_rr = part_at(2);
    w->part_aux = part_at(3);
    w->part_tt = part_at(4);
    w->st = reinterpret_cast<SysState*>(p + nv * vec + np * part);
    w->n_active = reinterpret_cast<int32_t*>(p + nv * vec + np * part + align256(sizeof(SysState) * nstate));
}

// A caller-fixed workspace block (the allocation-free entry point): the solve drivers
// carve their workspace from it instead of the handle's, and allocate nothing.
struct FixedWs {
    char* base;
    size_t bytes;
};

// G: the larger of the two grids (every partial array gets room for it).  nstate: the
// number of systems (batch, or the items of a SparseTensorList; < 0: batch).  With fx,
// the workspace is carved from fx's block (SLA_ERR_INVALID_ARG if it does not fit).
sla_status ensure_workspace(sla_csr* A, int64_t batch, int G, Workspace* w, int method = kMethodCG,
                            int64_t nstate = -1, const FixedWs* fx = nullptr)
{
    const int64_t n = A->n_rows;
    if (nstate < 0) nstate = batch;
    const size_t need = workspace_bytes(n, batch, G, method, nstate);
    if (fx) {
        if (need > fx->bytes)
            return fail(SLA_ERR_INVALID_ARG,
                        "the allocation-free solve needs %zu bytes of scratch here, more than its %zu",
                        need, fx->bytes);
        carve_workspace(fx->base, n, batch, G, w, method, nstate);
        return SLA_OK;
    }
    if (need > A->ws_bytes) {
        if (A->ws) {
            HIP_TRY(hipDeviceSynchronize());
            HIP_TRY(dev_free(A->ws));
            A->ws = nullptr;
            A->ws_bytes = 0;
        }
        sla_status s = dev_alloc(&A->ws, need);
        if (s != SLA_OK) return s;
        A->ws_bytes = need;
    }
    carve_workspace(static_cast<char*>(A->ws), n, batch, G, w, method, nstate);
    return SLA_OK;
}

sla_status check_opts(const sla_cg_opts* o)
{
    if (!o) return fail(SLA_ERR_INVALID_ARG, "opts is NULL");
    if (!(o->rtol >= 0.0) || !(o->atol >= 0.0))
        return fail(SLA_ERR_INVALID_ARG, "rtol and atol must be >= 0 (got %g, %g)", o->rtol, o->atol);
    if (o->max_iter < 0) return fail(SLA_ERR_INVALID_ARG, "max_iter must be >= 0");
    if (o->check_every < 0) return fail(SLA_ERR_INVALID_ARG, "check_every must be >= 0");
    if (o->flags & ~(SLA_FIXED_ITERS | SLA_JACOBI | SLA_BICGSTAB))
        return fail(SLA_ERR_INVALID_ARG, "unknown cg flags 0x%x", o->flags);
    if ((o->flags & SLA_JACOBI) && (o->flags & SLA_BICGSTAB))
        return fail(SLA_ERR_INVALID_ARG, "SLA_JACOBI and SLA_BICGSTAB cannot be combined");
    return SLA_OK;
}

// The transposed pattern, built once per handle.  Everything is built into local
// blocks first and handed to the handle only when all of it succeeded: a failed
// allocation or launch frees what this call allocated, so a later call starts clean.
sla_status ensure_transpose(sla_csr* A, hipStream_t s)
{
    if (A->has_t) return SLA_OK;
    void* rpt = nullptr;
    int32_t* colt = nullptr;
    int64_t* permt = nullptr;
    int16_t* c16t = nullptr;
    void* scratch = nullptr;
    auto release = [&](sla_status st) {
        (void)hipStreamSynchronize(s);   // no launch of this call may still use the blocks
        for (void* q : {rpt, static_cast<void*>(colt), static_cast<void*>(permt), static_cast<void*>(c16t), scratch})
            if (q) (void)dev_free(q);
        return st;
    };
    sla_status st;
    const size_t rpt_bytes = static_cast<size_t>(A->n_cols + 1) * (A->krp_bits == 64 ? 8 : 4);
    if ((st = dev_alloc(&rpt, std::max<size_t>(rpt_bytes, 8))) != SLA_OK) return release(st);
    if ((st = dev_alloc(reinterpret_cast<void**>(&colt), std::max<size_t>(4 * A->nnz, 4))) != SLA_OK)
        return release(st);
    if ((st = dev_alloc(reinterpret_cast<void**>(&permt), std::max<size_t>(8 * A->nnz, 8))) != SLA_OK)
        return release(st);
    if ((st = dev_alloc(&scratch, transpose_scratch_bytes(A->n_rows, A->n_cols, A->nnz))) != SLA_OK)
        return release(st);
    hipError_t e = timed(
        SLA_K_TRANSPOSE, s,
        [&] {
            return launch_transpose(A->krp, A->krp_bits, A->col, A->n_rows, A->n_cols, A->nnz, rpt, colt, permt,
                                    scratch, s);
        },
        false);
    if (e != hipSuccess) return release(fail(SLA_ERR_HIP, "transpose: %s", hipGetErrorString(e)));
    // analysis of the transposed pattern (also re-checks it)
    int32_t* d_chk = static_cast<int32_t*>(scratch);   // reuse: the scan data is no longer needed
    int32_t h[kChkCount] = {0, 0, 0, INT32_MAX, 0};
    e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipMemcpyAsync(d_chk, h, sizeof(h), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = launch_validate(rpt, A->krp_bits, colt, A->n_cols, A->n_rows, A->nnz, d_chk, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h, d_chk, sizeof(h), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return release(fail(SLA_ERR_HIP, "transpose analysis: %s", hipGetErrorString(e)));
    if (h[kChkErr] != 0)
        return release(fail(SLA_ERR_HIP, "internal error: transposed pattern failed validation (%d)", h[kChkErr]));
    // the transpose has the same spans |c - i|, so it gets offsets when A may have them
    if (A->c16_ok && A->krp_bits == 32) {
        if ((st = dev_alloc(reinterpret_cast<void**>(&c16t), sizeof(int16_t) * static_cast<size_t>(A->nnz))) !=
            SLA_OK)
            return release(st);
        e = launch_col16(static_cast<const int32_t*>(rpt), colt, c16t, A->n_cols, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return release(fail(SLA_ERR_HIP, "transposed column offsets: %s", hipGetErrorString(e)));
    }
    (void)dev_free(scratch);
    A->row_ptr_t = rpt;
    A->col_t = colt;
    A->perm_t = permt;
    A->col16_t = c16t;
    A->cap_t = choose_cap(h[kChkTileMax], h[kChkRowMax]);
    A->has_t = true;
    return SLA_OK;
}

// The 16-bit tile offsets of A's own pattern, built on first use when the handle did
// not build them at create (a banded handle, whose CG SpMV reads colb16).
sla_status ensure_col16(sla_csr* A, hipStream_t s)
{
    if (!A->c16_ok || A->col16) return SLA_OK;
    int16_t* c16 = nullptr;
    sla_status st = dev_alloc(reinterpret_cast<void**>(&c16), sizeof(int16_t) * static_cast<size_t>(A->nnz));
    if (st != SLA_OK) return st;
    hipError_t e = launch_col16(static_cast<const int32_t*>(A->krp), A->col, c16, A->n_rows, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(s);
        (void)dev_free(c16);
        return fail(SLA_ERR_HIP, "column offsets: %s", hipGetErrorString(e));
    }
    A->col16 = c16;
    return SLA_OK;
}

sla_status ensure_vals_t(sla_csr* A, int64_t batch, const double* vals, hipStream_t s, const double** out)
{
    const size_t need = sizeof(double) * static_cast<size_t>(A->nnz) * batch;
    if (need > A->vals_t_bytes) {
        if (A->vals_t) {
            HIP_TRY(hipDeviceSynchronize());
            HIP_TRY(dev_free(A->vals_t));
            A->vals_t = nullptr;
            A->vals_t_bytes = 0;
        }
        sla_status st = dev_alloc(reinterpret_cast<void**>(&A->vals_t), need);
        if (st != SLA_OK) return st;
        A->vals_t_bytes = need;
    }
    hipError_t e = timed(SLA_K_GATHER_VALS, s, [&] {
        return launch_gather_vals(A->perm_t, vals, A->vals_t, A->nnz, static_cast<int>(batch), s);
    });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "gather of transposed values: %s", hipGetErrorString(e));
    *out = A->vals_t;
    return SLA_OK;
}

// The diagonal layout of a banded handle (line stride A->band, 32-bit row pointers):
// the distinct offsets of its entries, ascending; with at most kDiaMax of them, their map
// and the per-row masks.  A pattern with more keeps the staged banded SpMV (dia_nd = 0).
sla_status build_dia(sla_csr* A, hipStream_t s)
{
    const int32_t S = static_cast<int32_t>(A->band);
    const int32_t* rp = static_cast<const int32_t*>(A->krp);
    uint32_t* d_codes = nullptr;
    sla_status st = dev_alloc(reinterpret_cast<void**>(&d_codes), 3 * sizeof(uint32_t));
    if (st != SLA_OK) return st;
    uint32_t h[3] = {0, 0, 0};
    hipError_t e = hipMemcpyAsync(d_codes, h, sizeof(h), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = launch_dia_codes(rp, A->col, A->n_rows, S, d_codes, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h, d_codes, sizeof(h), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    (void)dev_free(d_codes);
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "diagonal analysis: %s", hipGetErrorString(e));
    if (h[2] != 0) return SLA_OK;   // an entry off the band's diagonals (cannot happen for a banded handle)
    DiaMap m{};
    for (int c = 0; c <= kDiaCodes; ++c) m.d_of_code[c] = -1;
    int nd = 0;
    for (int c = 0; c < kDiaCodes; ++c) {
        const bool on = c < 32 ? ((h[0] >> c) & 1u) : ((h[1] >> (c - 32)) & 1u);
        if (!on) continue;
        if (nd == kDiaMax) return SLA_OK;   // too many diagonals: the staged banded SpMV
        m.d_of_code[c] = static_cast<int8_t>(nd);
        A->dia_b[nd] = static_cast<int8_t>(c / kDiaCodesPerBand - 1);
        A->dia_e[nd] = static_cast<int8_t>(c % kDiaCodesPerBand - kBandHalo);
        ++nd;
    }
    if (nd == 0) return SLA_OK;
    const bool m16 = nd > 8;
    void* mask = nullptr;
    if ((st = dev_alloc(&mask, (m16 ? 2 : 1) * static_cast<size_t>(A->n_rows))) != SLA_OK) return st;
    e = launch_dia_mask(rp, A->col, A->n_rows, S, m, mask, m16, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        (void)dev_free(mask);
        return fail(SLA_ERR_HIP, "diagonal masks: %s", hipGetErrorString(e));
    }
    A->dia_map = m;
    A->dia_mask = mask;
    A->dia_nd = nd;
    return SLA_OK;
}

// One CG solve (batch systems) on the pattern (row_ptr, col, cap) with values vals.
// Enqueue the iterations k = 0 .. max_iter (step(k) launches one iteration's kernels).
// Fixed-iteration mode enqueues them all.  Otherwise chunks of check_every (default
// 32) iterations go out with a copy of the device's running-systems counter after each
// chunk; two chunks are kept in flight and the loop ends once a copy reads 0.
template <class Step>
sla_status drive_cg(sla_csr* A, const CgArgs& a, const Workspace& w, const sla_cg_opts* o, hipStream_t s,
                    Step&& step)
{
    hipError_t e;
    if (a.fixed) {
        for (int64_t k = 0; k <= a.max_iter; ++k) {
            if ((e = step(k)) != hipSuccess) return fail(SLA_ERR_HIP, "cg launch: %s", hipGetErrorString(e));
        }
        return SLA_OK;
    }
    const int64_t chunk = o->check_every > 0 ? o->check_every : 32;
    int64_t k = 0;
    for (int64_t c = 0; k <= a.max_iter; ++c) {
        const int64_t kend = std::min<int64_t>(k + chunk, a.max_iter + 1);
        for (; k < kend; ++k) {
            if ((e = step(k)) != hipSuccess) return fail(SLA_ERR_HIP, "cg launch: %s", hipGetErrorString(e));
        }
        const int slot = static_cast<int>(c & 1);
        HIP_TRY(hipMemcpyAsync(A->flag_host + slot, w.n_active, sizeof(int32_t), hipMemcpyDeviceToHost, s));
        HIP_TRY(hipEventRecord(A->poll_ev[slot], s));
        if (c > 0) {
            HIP_TRY(hipEventSynchronize(A->poll_ev[slot ^ 1]));
            if (A->flag_host[slot ^ 1] == 0) break;   // every system has stopped
        }
    }
    return SLA_OK;
}

// The reordered pattern of the grouped kernels (once per handle; the pattern is 32-bit
// there).  Host copies of the pattern, the reverse Cuthill-McKee order, each new row's
// entries sorted by new column with the positions they came from.
sla_status ensure_reorder(sla_csr* A, hipStream_t s)
{
    if (A->g_reordered) return SLA_OK;
    const int64_t n = A->n_rows, nnz = A->nnz;
    std::vector<int32_t> rp(n + 1), col(std::max<int64_t>(nnz, 1));
    HIP_TRY(hipMemcpyAsync(rp.data(), A->krp, sizeof(int32_t) * (n + 1), hipMemcpyDeviceToHost, s));
    if (nnz > 0) HIP_TRY(hipMemcpyAsync(col.data(), A->col, sizeof(int32_t) * nnz, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    std::vector<int32_t> perm(n), inv(n), rp2(n + 1), col2(std::max<int64_t>(nnz, 1)), ep(std::max<int64_t>(nnz, 1));
    rcm_order(rp.data(), col.data(), n, perm.data());
    for (int64_t i = 0; i < n; ++i) inv[perm[i]] = static_cast<int32_t>(i);
    rp2[0] = 0;
    std::vector<std::pair<int32_t, int32_t>> row;
    for (int64_t i = 0; i < n; ++i) {
        const int32_t o = perm[i];
        row.clear();
        for (int32_t k = rp[o]; k < rp[o + 1]; ++k) row.emplace_back(inv[col[k]], k);
        std::sort(row.begin(), row.end());
        for (size_t j = 0; j < row.size(); ++j) {
            col2[rp2[i] + j] = row[j].first;
            ep[rp2[i] + j] = row[j].second;
        }
        rp2[i + 1] = rp2[i] + static_cast<int32_t>(row.size());
    }
    // bandwidth of the reordered pattern: the grouped SpMV's operand window needs every
    // column within g_halo rows of its row's tile
    int64_t bw = 0;
    for (int64_t i = 0; i < n; ++i)
        for (int32_t k = rp2[i]; k < rp2[i + 1]; ++k) bw = std::max<int64_t>(bw, std::abs(col2[k] - i));
    const int64_t halo = (bw + 63) / 64 * 64;
    A->g_halo = halo <= kGWinMaxHalo ? static_cast<int32_t>(halo) : 0;
    // with a window every column lies within halo + 63 rows of its tile's first row, so
    // the windowed SpMV reads these 16-bit offsets instead of the columns
    std::vector<int16_t> c16;
    if (A->g_halo > 0) {
        c16.resize(std::max<int64_t>(nnz, 1));
        for (int64_t i = 0; i < n; ++i)
            for (int32_t k = rp2[i]; k < rp2[i + 1]; ++k) c16[k] = static_cast<int16_t>(col2[k] - (i / 64) * 64);
    }
    auto release = [&]() {
        for (int32_t** q : {&A->g_rp, &A->g_col, &A->g_eperm, &A->g_perm}) {
            if (*q) (void)dev_free(*q);
            *q = nullptr;
        }
        if (A->g_col16) (void)dev_free(A->g_col16);
        A->g_col16 = nullptr;
    };
    release();   // nothing is left from an earlier attempt that failed
    sla_status st;
    if ((st = dev_alloc(reinterpret_cast<void**>(&A->g_rp), sizeof(int32_t) * (n + 1))) != SLA_OK ||
        (st = dev_alloc(reinterpret_cast<void**>(&A->g_col), sizeof(int32_t) * col2.size())) != SLA_OK ||
        (st = dev_alloc(reinterpret_cast<void**>(&A->g_eperm), sizeof(int32_t) * ep.size())) != SLA_OK ||
        (st = dev_alloc(reinterpret_cast<void**>(&A->g_perm), sizeof(int32_t) * n)) != SLA_OK ||
        (!c16.empty() &&
         (st = dev_alloc(reinterpret_cast<void**>(&A->g_col16), sizeof(int16_t) * c16.size())) != SLA_OK)) {
        release();
        return st;
    }
    HIP_TRY(hipMemcpyAsync(A->g_rp, rp2.data(), sizeof(int32_t) * (n + 1), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(A->g_col, col2.data(), sizeof(int32_t) * col2.size(), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(A->g_eperm, ep.data(), sizeof(int32_t) * ep.size(), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(A->g_perm, perm.data(), sizeof(int32_t) * n, hipMemcpyHostToDevice, s));
    if (!c16.empty())
        HIP_TRY(hipMemcpyAsync(A->g_col16, c16.data(), sizeof(int16_t) * c16.size(), hipMemcpyHostToDevice, s));
    HIP_TRY(hipStreamSynchronize(s));
    A->g_reordered = true;
    return SLA_OK;
}

// A pattern with no stored entries: the staged SpMV still issues its (clamped) entry
// loads on every path, so it gets readable stand-ins for the entry arrays (b, whose
// length n is nonzero whenever there is a tile to stage); nothing read is ever used.
void no_entries_standins(CgArgs& a, int64_t nnz)
{
    if (nnz > 0) return;
    a.vals = a.b;
    a.col = reinterpret_cast<const int32_t*>(a.b);
    a.col16 = reinterpret_cast<const int16_t*>(a.b);
}

// Grouped batch (kGroup systems interleaved per element): values into the grouped
// layout, then init / (p update, SpMV, update) per iteration / x back to the caller's
// layout.  The polling is run_cg's.  With the reordering on, the grouped kernels run on
// the reordered pattern: the values are gathered through the entry permutation, b and
// x through the row permutation, so the caller sees its own order.
sla_status run_cg_grouped(sla_csr* A, const void* row_ptr, const int32_t* col, int64_t batch, const double* vals,
                          const double* b, double* x, const sla_cg_opts* o, sla_cg_info* info, hipStream_t s)
{
    const int64_t n = A->n_rows;
    const int groups = static_cast<int>(batch / kGroup);
    const int64_t gtiles = std::max<int64_t>(1, (n + kBlock / kGroup - 1) / (kBlock / kGroup));
    // SpMV grid per group: with groups pinned to XCDs (groups % 8 == 0), the resident
    // workgroups of one XCD; otherwise an equal share of the GPU.
    const int gcap = static_cast<int64_t>(kBlock / kGroup) * A->row_max <= kGCapSmall ? kGCapSmall : kGCapLarge;
    const bool reorder = A->reorder_ok;
    if (reorder) {
        const sla_status st0 = ensure_reorder(A, s);
        if (st0 != SLA_OK) return st0;
    }
    // the operand window (k_gcg_spmv<..., true>) on a reordered pattern of small bandwidth
    const int32_t win = reorder && A->g_win_ok ? A->g_halo : 0;
    const int occ = cg_group_blocks_per_cu(gcap, win > 0);
    const bool pinned = groups >= 8 && groups % 8 == 0;
    int64_t P = pinned ? static_cast<int64_t>(A->n_cu / 8) * occ : (static_cast<int64_t>(A->n_cu) * occ) / groups;
    P = std::max<int64_t>(1, std::min<int64_t>(P, gtiles));
    // streaming kernels: about 16 tiles per workgroup (their start sums the partials)
    const int64_t Pu = std::max<int64_t>(1, std::min<int64_t>(64, (gtiles + 15) / 16));
    const bool jacobi = (o->flags & SLA_JACOBI) != 0;
    Workspace w;
    sla_status st = ensure_workspace(A, batch, static_cast<int>(std::max(P, Pu)), &w,
                                     jacobi ? kMethodJacobi : kMethodCG);
    if (st != SLA_OK) return st;
    const size_t xb = align256(sizeof(double) * static_cast<size_t>(n) * batch);
    const size_t need = xb + sizeof(double) * static_cast<size_t>(A->nnz) * batch;
    if (need > A->gws_bytes) {
        if (A->gws) {
            HIP_TRY(hipDeviceSynchronize());
            HIP_TRY(dev_free(A->gws));
            A->gws = nullptr;
            A->gws_bytes = 0;
        }
        if ((st = dev_alloc(&A->gws, need)) != SLA_OK) return st;
        A->gws_bytes = need;
    }
    double* xg = static_cast<double*>(A->gws);
    double* vg = reinterpret_cast<double*>(static_cast<char*>(A->gws) + xb);

    CgArgs a{};
    a.row_ptr = reorder ? static_cast<const void*>(A->g_rp) : row_ptr;
    a.col = reorder ? A->g_col : col;
    a.gperm = reorder ? A->g_perm : nullptr;
    a.vals = vg;
    a.b = b;
    a.x = x;
    a.r = w.r;
    a.p0 = w.p0;
    a.p1 = w.p1;
    a.q = w.q;
    a.part_sigma = w.part_sigma;
    a.part_rho = w.part_rho;
    a.part_rr = w.part_rr;
    a.part_aux = w.part_aux;
    a.z = w.z;       // Jacobi, grouped layout
    a.dg = w.dg;
    a.jacobi = jacobi ? 1 : 0;
    a.st = w.st;
    a.info = info;
    a.hist = o->residual_history;
    a.n_active = w.n_active;
    a.n = n;
    a.nnz = A->nnz;
    a.ntiles = gtiles;
    a.max_iter = o->max_iter;
    a.rtol = o->rtol;
    a.atol = o->atol;
    a.fixed = (o->flags & SLA_FIXED_ITERS) ? 1 : 0;
    a.G = static_cast<int32_t>(P);
    a.Gu = static_cast<int32_t>(Pu);
    a.batch = static_cast<int32_t>(batch);
    a.split = 1;
    a.groups = groups;
    a.cap = gcap;
    a.xg = xg;
    a.g_halo = win;
    a.g_col16 = win > 0 ? A->g_col16 : nullptr;

    hipError_t e = timed(SLA_K_GROUP_LAYOUT, s, [&] {
        return launch_group_vals(vals, vg, A->nnz, groups, reorder ? A->g_eperm : nullptr, s);
    });
    if (e == hipSuccess && jacobi) e = timed(SLA_K_CG_INIT, s, [&] { return launch_gcg(5, a, 0, s); });
    if (e == hipSuccess) e = timed(SLA_K_CG_INIT, s, [&] { return launch_gcg(0, a, 0, s); });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "grouped cg init: %s", hipGetErrorString(e));
    auto step = [&](int64_t k) -> hipError_t {
        hipError_t e0 = timed(SLA_K_CG_PUPD, s, [&] { return launch_gcg(1, a, k, s); });
        if (e0 != hipSuccess) return e0;
        e0 = timed(SLA_K_CG_SPMV, s, [&] { return launch_gcg(2, a, k, s); });
        if (e0 != hipSuccess || k >= a.max_iter) return e0;
        return timed(SLA_K_CG_UPDATE, s, [&] { return launch_gcg(3, a, k, s); });
    };
    if ((st = drive_cg(A, a, w, o, s, step)) != SLA_OK) return st;
    e = timed(SLA_K_GROUP_LAYOUT, s, [&] { return launch_gcg(4, a, 0, s); });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "grouped cg finish: %s", hipGetErrorString(e));
    return SLA_OK;
}

// SparseTensorList: per-system tables of the packed block-diagonal pattern (device
// arrays) and its one-dimensional grid, shared by every kernel of the solve.
struct ListPlan {
    const int32_t* wg;      // [items + 1] first workgroup of each system
    const int64_t* tiles;   // [items + 1] first tile of each system
    const int64_t* rend;    // [items] end of each system's real rows
    int32_t items;
    int32_t total_wg;
};

// band > 0: the pattern is banded with line stride `band` and takes the line-walking
// SpMV (LDS variant band_cap) on a persistent grid over blocks of lines of one strip.
// list: a SparseTensorList solve on the packed pattern (batch 1, plain or split SpMV).
// fx: the allocation-free entry point's scratch (nothing is allocated: no grouped
// layout, column offsets only where the handle already holds them).
sla_status run_cg(sla_csr* A, const void* row_ptr, const int32_t* col, int cap, int64_t band, int band_cap,
                  bool split, int64_t batch, const double* vals, const double* b, double* x, const sla_cg_opts* o,
                  sla_cg_info* info, hipStream_t s, const ListPlan* list = nullptr, const FixedWs* fx = nullptr)
{
    const bool jacobi = (o->flags & SLA_JACOBI) != 0;
    if (list) band = 0;
    if (!list && !fx && split && band == 0 && batch >= kGroupMinBatch && batch % kGroup == 0 &&
        A->krp_bits == 32 && A->nnz > 0 &&
        A->group_ok &&
        static_cast<int64_t>(kBlock / kGroup) * A->row_max <= kGCapLarge && row_ptr == A->krp)
        return run_cg_grouped(A, row_ptr, col, batch, vals, b, x, o, info, s);
    const int64_t n = A->n_rows;
    const int64_t ntiles = (n + kTile - 1) / kTile;
    // Grid of the plain SpMV (also the base of the update kernel's grid).
    if (band > 0) split = false;
    const int Gp = blocks_per_system(A, ntiles, batch, cg_blocks_per_cu(A->krp_bits, cap, n, split));
    int G = Gp, band_block = 0;
    int64_t band_lines = 0;
    // The diagonal layout (k_cg_spmv_dia) serves a banded handle's own pattern whenever
    // it exists; the allocation-free entry point keeps the staged banded SpMV (the layout's
    // values need a buffer).
    const bool dia = band > 0 && !list && !fx && A->dia_nd > 0 && row_ptr == A->krp && col == A->col;
    if (band > 0) {
        // Persistent grid over blocks of band_block lines of one strip (k_cg_spmv_band,
        // k_cg_spmv_dia): blocks of up to kBandBlockLines lines, shorter when needed to
        // give every workgroup of the grid a block.
        const int64_t strips = (band + kTile - 1) / kTile;
        band_lines = (n + band - 1) / band;
        const int64_t spmv_bytes = (12 * A->nnz + 52 * n) * batch;   // values, columns, rows, six vectors
        int per_cu = dia ? cg_dia_blocks_per_cu(A->dia_nd) : cg_band_blocks_per_cu(band_cap);
        if (spmv_bytes > kBandStreamBytes) per_cu = std::min(per_cu, dia ? kDiaBlocksPerCu : kBandBlocksPerCu);
        const int64_t target = std::max<int64_t>(1, (static_cast<int64_t>(A->n_cu) * per_cu) / batch);
        const int64_t bl = std::max<int64_t>(4, std::min<int64_t>(kBandBlockLines, strips * band_lines / target));
        // Within [bl / 2, bl], the block length whose busiest workgroup walks the fewest
        // lines (ties to the longer blocks, which restart the pipeline less often): blocks
        // that do not divide evenly over the grid leave most workgroups idle at the end.
        int64_t best_b = 0, best_cost = 0;
        for (int64_t bb = bl; bb >= std::max<int64_t>(4, bl / 2); --bb) {
            const int64_t nb = strips * ((band_lines + bb - 1) / bb);
            const int64_t g = std::min<int64_t>(nb, target);
            const int64_t cost = ((nb + g - 1) / g) * bb;
            if (best_b == 0 || cost < best_cost) best_b = bb, best_cost = cost;
        }
        band_block = static_cast<int>(std::min<int64_t>(band_lines, best_b));
        const int64_t nblk = strips * ((band_lines + band_block - 1) / band_block);
        G = static_cast<int>(std::min<int64_t>(nblk, target));
        cap = band_cap;
    }
    // The update kernel streams 24 B per row and starts by summing all of the SpMV's
    // partials: about 8 tiles per workgroup balances its start-up cost against the
    // memory parallelism it needs (a smaller grid for small systems, the plain SpMV's
    // full-occupancy grid for large ones; at 1M rows 8 measured 7.2-7.4 us per launch,
    // 6 7.7, 12 8.1, 16 8.2).
    int Gu = Gp;
    if (batch < 8 || batch % 8 != 0) {
        int64_t g = ((ntiles + 7) / 8 + 7) & ~int64_t(7);
        Gu = static_cast<int>(std::max<int64_t>(8, std::min<int64_t>(Gp, g)));
        if (Gu > ntiles) Gu = Gp;
    }
    // The 16-byte update kernel (k_cg_update_wide) serves every per-system solve whose
    // vectors are 16-byte aligned: one system, or an even n (the caller's b, read as r_0,
    // must be aligned too).  Systems that stream from HBM give it exactly 3 workgroups
    // per CU, whatever the plain SpMV's occupancy: at 169M rows 684 us per launch against
    // 782 us for the 8-tile kernel on one box (1024 workgroups: 701 us; 2048: 810 us); at
    // 1M rows the 8-tile grid stays best for it too (6.6 us against 7.2 us for the
    // 8-tile kernel).
    const bool wide = !list && !(batch >= 8 && batch % 8 == 0) && (batch == 1 || n % 2 == 0) &&
                      (reinterpret_cast<uintptr_t>(b) & 15) == 0;
    const bool streaming = (12 * A->nnz + 52 * n) * batch > kBandStreamBytes;
    if (wide && streaming && batch == 1) Gu = 3 * A->n_cu;
    if (list) G = Gu = list->total_wg;   // one grid and one partial slot per workgroup
    Workspace w;
    sla_status st = ensure_workspace(A, batch, std::max(G, Gu), &w, jacobi ? kMethodJacobi : kMethodCG,
                                     list ? list->items : -1, fx);
    if (st != SLA_OK) return st;
    if (!fx && band == 0 && col == A->col && (st = ensure_col16(A, s)) != SLA_OK) return st;
    if (dia) {
        const size_t need = sizeof(double) * static_cast<size_t>(A->dia_nd) * n * batch;
        if (need > A->dia_vals_bytes) {
            if (A->dia_vals) {
                HIP_TRY(hipDeviceSynchronize());
                HIP_TRY(dev_free(A->dia_vals));
                A->dia_vals = nullptr;
                A->dia_vals_bytes = 0;
            }
            if ((st = dev_alloc(reinterpret_cast<void**>(&A->dia_vals), need)) != SLA_OK) return st;
            A->dia_vals_bytes = need;
        }
        hipError_t e = timed(SLA_K_GROUP_LAYOUT, s, [&] {
            return launch_dia_vals(static_cast<const int32_t*>(A->krp), A->col, vals, n, A->nnz,
                                   static_cast<int32_t>(band), A->dia_map, A->dia_nd, static_cast<int>(batch),
                                   A->dia_vals, s);
        });
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "diagonal layout of the values: %s", hipGetErrorString(e));
    }

    CgArgs a{};
    a.row_ptr = row_ptr;
    a.col = col;
    a.col16 = (col == A->col && row_ptr == A->krp) ? A->col16 : (col == A->col_t ? A->col16_t : nullptr);
    if (band > 0) a.col16 = A->colb16;   // the banded SpMV's window-relative offsets, or none
    a.vals = vals;
    a.b = b;
    no_entries_standins(a, A->nnz);
    a.x = x;
    a.r = w.r;
    a.p0 = w.p0;
    a.p1 = w.p1;
    a.q = w.q;
    a.part_sigma = w.part_sigma;
    a.part_rho = w.part_rho;
    a.part_rr = w.part_rr;
    a.part_aux = w.part_aux;
    a.z = w.z;
    a.dg = w.dg;
    a.jacobi = jacobi ? 1 : 0;
    a.st = w.st;
    a.info = info;
    a.hist = o->residual_history;
    a.n_active = w.n_active;
    a.n = n;
    a.nnz = A->nnz;
    a.ntiles = ntiles;
    a.max_iter = o->max_iter;
    a.rtol = o->rtol;
    a.atol = o->atol;
    a.fixed = (o->flags & SLA_FIXED_ITERS) ? 1 : 0;
    a.G = G;
    a.Gu = Gu;
    a.batch = static_cast<int32_t>(batch);
    a.xcd_remap = 1;
    a.sys_per_xcd = (batch >= 8 && batch % 8 == 0) ? 1 : 0;
    a.split = split ? 1 : 0;
    // systems far beyond the caches: the update pass streams with the non-temporal
    // hint (measured 5 % faster at 169M rows; slower where the 256 MB cache holds the
    // working set across iterations)
    a.stream_nt = streaming ? 1 : 0;
    a.wide_update = wide ? 1 : 0;
    a.band_block = band_block;
    a.band_stride = band;
    a.band_lines = band_lines;
    if (dia) {
        a.dia_vals = A->dia_vals;
        a.dia_mask = A->dia_mask;
        a.dia_nd = A->dia_nd;
        a.dia_shift = (A->dia_align && band % 16 == 8) ? 8 : 0;
        for (int d = 0; d < kDiaMax; ++d) {
            a.dia_b[d] = d < A->dia_nd ? A->dia_b[d] : 0;
            a.dia_e[d] = d < A->dia_nd ? A->dia_e[d] : 0;
            a.dia_v[d] = A->dia_vals + static_cast<size_t>(std::min(d, A->dia_nd - 1)) * n;
        }
    }
    if (list) {
        a.list_wg = list->wg;
        a.list_tiles = list->tiles;
        a.list_rend = list->rend;
        a.list_items = list->items;
        a.sys_per_xcd = 0;
        a.xcd_remap = 0;
    }
    const int rp_bits = A->krp_bits;   // A and its transpose use the same row-pointer width

    hipError_t e = hipSuccess;
    if (a.jacobi) e = timed(SLA_K_CG_INIT, s, [&] { return launch_cg_diag(a, rp_bits, s); });
    if (e == hipSuccess) e = timed(SLA_K_CG_INIT, s, [&] { return launch_cg_init(a, s); });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "cg init launch: %s", hipGetErrorString(e));

    auto step = [&](int64_t k) -> hipError_t {
        if (a.split) {
            hipError_t e0 = timed(SLA_K_CG_PUPD, s, [&] { return launch_cg_pupd(a, k, s); });
            if (e0 != hipSuccess) return e0;
        }
        hipError_t e1 = timed(SLA_K_CG_SPMV, s, [&] { return launch_cg_spmv(a, k, rp_bits, cap, s); });
        if (e1 != hipSuccess || k >= a.max_iter) return e1;
        return timed(SLA_K_CG_UPDATE, s, [&] { return launch_cg_update(a, k, s); });
    };
    return drive_cg(A, a, w, o, s, step);
}

// BiCGStab on the pattern (row_ptr, col; LDS variant cap) with values vals: init, then
// per iteration the p update, v = A p, s, t = A s and the update.  The SpMV grid fills
// the GPU once as the CG SpMV's does, the streaming kernels take about 8 tiles per
// workgroup (as CG's update; at 1M rows 10.3 us per launch against 11.0 with 16); the
// polling is run_cg's.
sla_status run_bicgstab(sla_csr* A, const void* row_ptr, const int32_t* col, int cap, int64_t batch,
                        const double* vals, const double* b, double* x, const sla_cg_opts* o, sla_cg_info* info,
                        hipStream_t s, const FixedWs* fx = nullptr)
{
    const int64_t n = A->n_rows;
    const int64_t ntiles = (n + kTile - 1) / kTile;
    const int rp_bits = A->krp_bits;   // A and its transpose use the same row-pointer width
    const int G = blocks_per_system(A, ntiles, batch, bs_blocks_per_cu(rp_bits, cap, n));
    int Gu = G;
    if (batch < 8 || batch % 8 != 0) {
        int64_t g = ((ntiles + 7) / 8 + 7) & ~int64_t(7);
        Gu = static_cast<int>(std::max<int64_t>(8, std::min<int64_t>(G, g)));
        if (Gu > ntiles) Gu = G;
    }
    Workspace w;
    sla_status st = ensure_workspace(A, batch, std::max(G, Gu), &w, kMethodBiCGStab, -1, fx);
    if (st != SLA_OK) return st;
    if (!fx && col == A->col && (st = ensure_col16(A, s)) != SLA_OK) return st;

    CgArgs a{};
    a.row_ptr = row_ptr;
    a.col = col;
    a.col16 = (col == A->col && row_ptr == A->krp) ? A->col16 : (col == A->col_t ? A->col16_t : nullptr);
    a.vals = vals;
    a.b = b;
    no_entries_standins(a, A->nnz);
    a.x = x;
    a.r = w.r;
    a.p0 = w.p0;   // p
    a.p1 = w.p1;   // s
    a.q = w.q;     // v
    a.z = w.z;     // t
    a.part_sigma = w.part_sigma;
    a.part_rho = w.part_rho;
    a.part_rr = w.part_rr;
    a.part_aux = w.part_aux;
    a.part_tt = w.part_tt;
    a.st = w.st;
    a.info = info;
    a.hist = o->residual_history;
    a.n_active = w.n_active;
    a.n = n;
    a.nnz = A->nnz;
    a.ntiles = ntiles;
    a.max_iter = o->max_iter;
    a.rtol = o->rtol;
    a.atol = o->atol;
    a.fixed = (o->flags & SLA_FIXED_ITERS) ? 1 : 0;
    a.G = G;
    a.Gu = Gu;
    a.batch = static_cast<int32_t>(batch);
    a.xcd_remap = 1;
    a.sys_per_xcd = (batch >= 8 && batch % 8 == 0) ? 1 : 0;
    a.split = 1;

    hipError_t e = timed(SLA_K_BS_VEC, s, [&] { return launch_bs(0, a, 0, rp_bits, cap, s); });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "bicgstab init launch: %s", hipGetErrorString(e));
    auto step = [&](int64_t k) -> hipError_t {
        hipError_t e0 = timed(SLA_K_BS_VEC, s, [&] { return launch_bs(1, a, k, rp_bits, cap, s); });
        if (e0 != hipSuccess || k >= a.max_iter) return e0;
        static const int kOrder[4] = {2, 3, 4, 5};
        for (int which : kOrder) {
            const int kid = (which == 2 || which == 4) ? SLA_K_BS_SPMV : SLA_K_BS_VEC;
            e0 = timed(kid, s, [&] { return launch_bs(which, a, k, rp_bits, cap, s); });
            if (e0 != hipSuccess) return e0;
        }
        return hipSuccess;
    };
    return drive_cg(A, a, w, o, s, step);
}

// Line stride of a banded pattern, or 0.  Banded: square with n < 2^29 and nnz < 2^31
// (the kernel uses 32-bit offsets and the 32-bit row pointers), every entry within
// kBandHalo of the diagonal or within kBandHalo below the largest distance S, whole
// windows of kTile rows fit the largest LDS variant, and S at least the minimum stride
// (default 2048; environment SLA_BAND_MIN_STRIDE overrides it, read at each create).
// Below that stride the plain SpMV's gathers already stay in L2.
int64_t band_stride_of(int64_t n_rows, int64_t n_cols, int64_t nnz, int32_t row_max, int32_t far_min,
                       int32_t far_max)
{
    int64_t min_stride = 2048;
    if (const char* env = std::getenv("SLA_BAND_MIN_STRIDE")) {
        char* end = nullptr;
        const long long v = std::strtoll(env, &end, 10);
        if (end != env && v > 0) min_stride = v;
    }
    const int64_t S = far_max;
    // (an empty pattern never takes the banded kernel: its staging clamps to entry nnz - 1)
    if (n_rows != n_cols || n_rows >= (int64_t(1) << 29) || nnz < 1 || nnz >= (int64_t(1) << 31) || S <= 0) return 0;
    if (far_min < S - kBandHalo) return 0;
    if (S < kTile + 2 * kBandHalo || S < min_stride) return 0;
    if (static_cast<int64_t>(kTile) * row_max > kCapLarge) return 0;
    return S;
}

sla_status check_common(const sla_csr* A, int64_t batch)
{
    if (!A) return fail(SLA_ERR_INVALID_ARG, "handle is NULL");
    if (batch < 1 || batch > 65535) return fail(SLA_ERR_INVALID_ARG, "batch must be in [1, 65535] (got %lld)",
                                               static_cast<long long>(batch));
    return check_device(A);
}

}  // namespace

// =====================================================================================
extern "C" {

const char* sla_status_string(sla_status s)
{
    switch (s) {
    case SLA_OK: return "SLA_OK";
    case SLA_ERR_INVALID_ARG: return "SLA_ERR_INVALID_ARG";
    case SLA_ERR_INVALID_CSR: return "SLA_ERR_INVALID_CSR";
    case SLA_ERR_UNSUPPORTED: return "SLA_ERR_UNSUPPORTED";
    case SLA_ERR_OOM: return "SLA_ERR_OOM";
    case SLA_ERR_HIP: return "SLA_ERR_HIP";
    }
    return "SLA_UNKNOWN_STATUS";
}

const char* sla_last_error(void) { return g_err; }

int32_t sla_version(void) { return 100; }

sla_status sla_csr_create(sla_csr** out, int64_t n_rows, int64_t n_cols, int64_t nnz, const void* d_row_ptr,
                          int32_t row_ptr_bits, const int32_t* d_col_idx, uint32_t flags, void* stream)
{
    if (!out) return fail(SLA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (n_rows < 0 || n_cols < 0 || nnz < 0) return fail(SLA_ERR_INVALID_ARG, "negative size");
    if (n_rows >= (int64_t(1) << 31) || n_cols >= (int64_t(1) << 31))
        return fail(SLA_ERR_INVALID_ARG, "n_rows and n_cols must be < 2^31");
    if (row_ptr_bits != 32 && row_ptr_bits != 64)
        return fail(SLA_ERR_INVALID_ARG, "row_ptr_bits must be 32 or 64 (got %d)", row_ptr_bits);
    if (row_ptr_bits == 32 && nnz >= (int64_t(1) << 31))
        return fail(SLA_ERR_INVALID_ARG, "nnz >= 2^31 needs 64-bit row pointers");
    if (!d_row_ptr) return fail(SLA_ERR_INVALID_ARG, "row_ptr is NULL");
    if (!d_col_idx && nnz > 0) return fail(SLA_ERR_INVALID_ARG, "col_idx is NULL");
    if (flags & ~(SLA_SYMMETRIC | SLA_EAGER_TRANSPOSE)) return fail(SLA_ERR_INVALID_ARG, "unknown csr flags 0x%x", flags);
    if ((flags & SLA_SYMMETRIC) && n_rows != n_cols)
        return fail(SLA_ERR_INVALID_ARG, "SLA_SYMMETRIC needs a square matrix");
    hipStream_t s = static_cast<hipStream_t>(stream);

    sla_csr* A = new (std::nothrow) sla_csr();
    if (!A) return fail(SLA_ERR_OOM, "host allocation failed");
    A->n_rows = n_rows;
    A->n_cols = n_cols;
    A->nnz = nnz;
    A->rp_bits = row_ptr_bits;
    A->flags = flags;
    A->row_ptr = d_row_ptr;
    A->col = d_col_idx;
    auto bail = [&](sla_status st) {
        sla_csr_destroy(A);
        return st;
    };
    if (hipGetDevice(&A->device) != hipSuccess) return bail(fail(SLA_ERR_HIP, "hipGetDevice failed"));
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, A->device) == hipSuccess && ncu > 0)
        A->n_cu = ncu;
    if (hipHostMalloc(reinterpret_cast<void**>(&A->flag_host), 2 * sizeof(int32_t), hipHostMallocDefault) !=
        hipSuccess)
        return bail(fail(SLA_ERR_OOM, "pinned host allocation failed"));
    A->flag_host[0] = A->flag_host[1] = -1;
    for (int i = 0; i < 2; ++i)
        if (hipEventCreateWithFlags(&A->poll_ev[i], hipEventDisableTiming) != hipSuccess)
            return bail(fail(SLA_ERR_HIP, "hipEventCreate failed"));

    // Validation and pattern analysis: one device pass, one synchronisation.
    int32_t* d_chk = nullptr;
    sla_status st = dev_alloc(reinterpret_cast<void**>(&d_chk), kChkCount * sizeof(int32_t));
    if (st != SLA_OK) return bail(st);
    int32_t h[kChkCount] = {0, 0, 0, INT32_MAX, 0};
    hipError_t e = hipMemcpyAsync(d_chk, h, sizeof(h), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = launch_validate(d_row_ptr, row_ptr_bits, d_col_idx, n_rows, n_cols, nnz, d_chk, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h, d_chk, sizeof(h), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    (void)dev_free(d_chk);
    if (e != hipSuccess) return bail(fail(SLA_ERR_HIP, "CSR validation: %s", hipGetErrorString(e)));
    if (h[kChkErr] != 0) {
        const int c = h[kChkErr];
        const char* why = (c & 1) ? "row_ptr[0] != 0 or row_ptr[n_rows] != nnz"
                          : (c & 2) ? "row_ptr is not non-decreasing within [0, nnz]"
                          : (c & 4) ? "a column index is out of [0, n_cols)"
                                    : "columns are not strictly ascending within a row";
        return bail(fail(SLA_ERR_INVALID_CSR, "invalid CSR: %s (code %d)", why, c));
    }
    A->tile_max = h[kChkTileMax];
    A->row_max = h[kChkRowMax];
    A->cap = choose_cap(h[kChkTileMax], h[kChkRowMax]);
    A->band = band_stride_of(n_rows, n_cols, nnz, h[kChkRowMax], h[kChkFarMin], h[kChkFarMax]);
    A->band_cap = choose_cap(kTile * std::max<int32_t>(h[kChkRowMax], 1), 0);
    A->split = A->band == 0 && h[kChkFarMax] >= kSplitMinSpan;
    if (const char* env = std::getenv("SLA_CG_SCHEDULE")) {   // "fused" or "split" overrides the choice
        if (std::strcmp(env, "fused") == 0) A->split = false;
        if (std::strcmp(env, "split") == 0) A->split = A->band == 0;
    }
    if (const char* env = std::getenv("SLA_CG_GROUPED")) A->group_ok = std::strcmp(env, "0") != 0;
    if (const char* env = std::getenv("SLA_CG_REORDER")) A->reorder_ok = std::strcmp(env, "0") != 0;
    if (const char* env = std::getenv("SLA_GCG_WINDOW")) A->g_win_ok = std::strcmp(env, "0") != 0;
    A->krp = d_row_ptr;
    A->krp_bits = row_ptr_bits;
    if (row_ptr_bits == 64 && nnz < (int64_t(1) << 31)) {
        if ((st = dev_alloc(&A->rp_owned, sizeof(int32_t) * static_cast<size_t>(n_rows + 1))) != SLA_OK)
            return bail(st);
        e = launch_narrow_rp(static_cast<const int64_t*>(d_row_ptr), static_cast<int32_t*>(A->rp_owned), n_rows + 1,
                             s);
        if (e != hipSuccess) return bail(fail(SLA_ERR_HIP, "row pointer copy: %s", hipGetErrorString(e)));
        A->krp = A->rp_owned;
        A->krp_bits = 32;
    }
    bool c16 = A->krp_bits == 32 && n_rows == n_cols && n_rows < (int64_t(1) << 29) && nnz > 0 &&
               std::max<int32_t>(h[kChkFarMax], kBandHalo) <= kCol16MaxSpan;
    if (const char* env = std::getenv("SLA_COL16")) c16 = c16 && std::strcmp(env, "0") != 0;
    A->c16_ok = c16;
    const bool cb16 = c16 && A->band > 0 && A->band <= kCol16MaxSpan;
    if (c16 && !cb16) {   // a banded handle builds the tile offsets on first use only
        if ((st = dev_alloc(reinterpret_cast<void**>(&A->col16), sizeof(int16_t) * static_cast<size_t>(nnz))) !=
            SLA_OK)
            return bail(st);
        e = launch_col16(static_cast<const int32_t*>(A->krp), d_col_idx, A->col16, n_rows, s);
        if (e != hipSuccess) return bail(fail(SLA_ERR_HIP, "column offsets: %s", hipGetErrorString(e)));
    }
    if (cb16) {
        if ((st = dev_alloc(reinterpret_cast<void**>(&A->colb16), sizeof(int16_t) * static_cast<size_t>(nnz))) !=
            SLA_OK)
            return bail(st);
        e = launch_colb16(static_cast<const int32_t*>(A->krp), d_col_idx, A->colb16, n_rows,
                          static_cast<int32_t>(A->band), s);
        if (e != hipSuccess) return bail(fail(SLA_ERR_HIP, "band column offsets: %s", hipGetErrorString(e)));
    }
    if (A->band > 0 && A->krp_bits == 32) {
        bool dia = true;
        if (const char* env = std::getenv("SLA_DIA")) dia = std::strcmp(env, "0") != 0;
        if (const char* env = std::getenv("SLA_DIA_ALIGN")) A->dia_align = std::strcmp(env, "0") != 0;
        if (dia && (st = build_dia(A, s)) != SLA_OK) return bail(st);
    }
    if (A->rp_owned || A->col16 || A->colb16 || A->dia_mask) {   // the handle may next be used on another stream
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return bail(fail(SLA_ERR_HIP, "create: %s", hipGetErrorString(e)));
    }
    if ((flags & SLA_EAGER_TRANSPOSE) && !(flags & SLA_SYMMETRIC)) {
        std::lock_guard<std::mutex> lk(A->mu);
        if ((st = ensure_transpose(A, s)) != SLA_OK) return bail(st);
    }
    *out = A;
    return SLA_OK;
}

sla_status sla_csr_destroy(sla_csr* A)
{
    if (!A) return SLA_OK;
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != A->device) (void)hipSetDevice(A->device);
    (void)hipDeviceSynchronize();
    if (A->ws) (void)dev_free(A->ws);
    if (A->gws) (void)dev_free(A->gws);
    if (A->vals_t) (void)dev_free(A->vals_t);
    if (A->row_ptr_t) (void)dev_free(A->row_ptr_t);
    if (A->col_t) (void)dev_free(A->col_t);
    if (A->perm_t) (void)dev_free(A->perm_t);
    if (A->rp_owned) (void)dev_free(A->rp_owned);
    if (A->col16) (void)dev_free(A->col16);
    if (A->col16_t) (void)dev_free(A->col16_t);
    if (A->colb16) (void)dev_free(A->colb16);
    if (A->dia_mask) (void)dev_free(A->dia_mask);
    if (A->dia_vals) (void)dev_free(A->dia_vals);
    if (A->flag_host) (void)hipHostFree(A->flag_host);
    if (A->eig_ws) (void)dev_free(A->eig_ws);
    if (A->g_rp) (void)dev_free(A->g_rp);
    if (A->g_col) (void)dev_free(A->g_col);
    if (A->g_eperm) (void)dev_free(A->g_eperm);
    if (A->g_perm) (void)dev_free(A->g_perm);
    if (A->g_col16) (void)dev_free(A->g_col16);
    if (A->eig_host) (void)hipHostFree(A->eig_host);
    if (A->lob_ws) (void)dev_free(A->lob_ws);
    if (A->lob_host) (void)hipHostFree(A->lob_host);
    if (A->lob_res) (void)hipHostFree(A->lob_res);
    for (int i = 0; i < 2; ++i)
        if (A->poll_ev[i]) (void)hipEventDestroy(A->poll_ev[i]);
    if (prev >= 0 && prev != A->device) (void)hipSetDevice(prev);
    delete A;
    return SLA_OK;
}

sla_status sla_csr_analysis(const sla_csr* A, int32_t* row_max, int32_t* tile_max, int32_t* spmv_cap,
                            int64_t* band_stride, int32_t* cg_split)
{
    if (!A) return fail(SLA_ERR_INVALID_ARG, "handle is NULL");
    if (row_max) *row_max = A->row_max;
    if (tile_max) *tile_max = A->tile_max;
    if (spmv_cap) *spmv_cap = std::min(A->band > 0 ? A->band_cap : A->cap, kCapLarge);
    if (band_stride) *band_stride = A->band;
    if (cg_split) *cg_split = A->split ? 1 : 0;
    return SLA_OK;
}

sla_status sla_csr_col_bits(const sla_csr* A, int32_t* col_bits)
{
    if (!A) return fail(SLA_ERR_INVALID_ARG, "handle is NULL");
    if (col_bits) *col_bits = A->c16_ok ? 16 : 32;
    return SLA_OK;
}

sla_status sla_csr_diagonals(const sla_csr* A, int32_t* n_diagonals)
{
    if (!A) return fail(SLA_ERR_INVALID_ARG, "handle is NULL");
    if (n_diagonals) *n_diagonals = A->dia_nd;
    return SLA_OK;
}

sla_status sla_csr_group_window(const sla_csr* A, int32_t* halo_rows)
{
    if (!A) return fail(SLA_ERR_INVALID_ARG, "handle is NULL");
    if (halo_rows) *halo_rows = (A->g_reordered && A->reorder_ok && A->g_win_ok) ? A->g_halo : 0;
    return SLA_OK;
}

sla_status sla_csr_info(const sla_csr* A, int64_t* n_rows, int64_t* n_cols, int64_t* nnz, int32_t* row_ptr_bits,
                        uint32_t* flags, int64_t* workspace_bytes_out)
{
    if (!A) return fail(SLA_ERR_INVALID_ARG, "handle is NULL");
    if (n_rows) *n_rows = A->n_rows;
    if (n_cols) *n_cols = A->n_cols;
    if (nnz) *nnz = A->nnz;
    if (row_ptr_bits) *row_ptr_bits = A->rp_bits;
    if (flags) *flags = A->flags;
    if (workspace_bytes_out) {
        int64_t tb = 0;
        if (A->has_t)
            tb = (A->n_cols + 1) * (A->krp_bits == 64 ? 8 : 4) + 12 * A->nnz;
        if (A->rp_owned) tb += 4 * (A->n_rows + 1);
        if (A->col16) tb += 2 * A->nnz;
        if (A->col16_t) tb += 2 * A->nnz;
        if (A->colb16) tb += 2 * A->nnz;
        if (A->dia_mask) tb += (A->dia_nd > 8 ? 2 : 1) * A->n_rows;
        *workspace_bytes_out = static_cast<int64_t>(A->ws_bytes + A->vals_t_bytes + A->dia_vals_bytes) + tb;
    }
    return SLA_OK;
}

sla_status sla_matvec(const sla_csr* Ac, int64_t batch, const double* d_vals, const double* d_x, double* d_y,
                      void* stream)
{
    sla_status st = check_common(Ac, batch);
    if (st != SLA_OK) return st;
    if ((!d_vals && Ac->nnz > 0) || (!d_x && Ac->n_cols > 0) || (!d_y && Ac->n_rows > 0))
        return fail(SLA_ERR_INVALID_ARG, "NULL array");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed(SLA_K_MATVEC, s, [&] {
        return launch_matvec(Ac->krp, Ac->krp_bits, Ac->col, d_vals, d_x, d_y, Ac->n_rows, Ac->nnz, Ac->n_cols,
                             static_cast<int>(batch), Ac->cap, s);
    });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "matvec launch: %s", hipGetErrorString(e));
    return SLA_OK;
}

sla_status sla_matvec_backward(const sla_csr* Ac, int64_t batch, const double* d_vals, const double* d_x,
                               const double* d_gy, double* d_gx, double* d_gvals, void* stream)
{
    sla_status st = check_common(Ac, batch);
    if (st != SLA_OK) return st;
    if (!d_gy && Ac->n_rows > 0) return fail(SLA_ERR_INVALID_ARG, "gy is NULL");
    if (d_gx && !d_vals && Ac->nnz > 0) return fail(SLA_ERR_INVALID_ARG, "vals is NULL");
    if (d_gvals && !d_x && Ac->n_cols > 0) return fail(SLA_ERR_INVALID_ARG, "x is NULL");
    sla_csr* A = const_cast<sla_csr*>(Ac);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lk(A->mu);
    if (d_gx) {
        hipError_t e;
        if (A->flags & SLA_SYMMETRIC) {
            e = timed(SLA_K_MATVEC, s, [&] {
                return launch_matvec(A->krp, A->krp_bits, A->col, d_vals, d_gy, d_gx, A->n_rows, A->nnz,
                                     A->n_cols, static_cast<int>(batch), A->cap, s);
            });
        } else {
            if ((st = ensure_transpose(A, s)) != SLA_OK) return st;
            const double* vt = nullptr;
            if ((st = ensure_vals_t(A, batch, d_vals, s, &vt)) != SLA_OK) return st;
            e = timed(SLA_K_MATVEC, s, [&] {
                return launch_matvec(A->row_ptr_t, A->krp_bits, A->col_t, vt, d_gy, d_gx, A->n_cols, A->nnz,
                                     A->n_rows, static_cast<int>(batch), A->cap_t, s);
            });
        }
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "matvec_backward launch: %s", hipGetErrorString(e));
    }
    if (d_gvals) {
        hipError_t e = timed(SLA_K_PATTERN_OUTER, s, [&] {
            return launch_pattern_outer(A->krp, A->krp_bits, A->col, 1.0, d_gy, A->n_rows, d_x, A->n_cols,
                                        d_gvals, A->n_rows, A->nnz, static_cast<int>(batch), s);
        });
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "pattern outer launch: %s", hipGetErrorString(e));
    }
    return SLA_OK;
}

}  // extern "C"

namespace {

// A 0 x 0 system: every one converges with 0 iterations (x and lambda are empty).
sla_status empty_solve_info(int64_t batch, sla_cg_info* d_info, hipStream_t s)
{
    std::vector<sla_cg_info> h(static_cast<size_t>(batch));
    for (auto& i : h) {
        i.iterations = 0;
        i.res_norm = 0.0;
        i.rhs_norm = 0.0;
        i.state = SLA_CONVERGED;
        i.reserved = 0;
    }
    HIP_TRY(hipMemcpyAsync(d_info, h.data(), sizeof(sla_cg_info) * h.size(), hipMemcpyHostToDevice, s));
    HIP_TRY(hipStreamSynchronize(s));   // h is pageable and local
    return SLA_OK;
}

}  // namespace

extern "C" {

sla_status sla_solve(const sla_csr* Ac, int64_t batch, const double* d_vals, const double* d_b, double* d_x,
                     const sla_cg_opts* opts, sla_cg_info* d_info, void* stream)
{
    sla_status st = check_common(Ac, batch);
    if (st != SLA_OK) return st;
    if (Ac->n_rows != Ac->n_cols) return fail(SLA_ERR_UNSUPPORTED, "solve needs a square matrix");
    if ((st = check_opts(opts)) != SLA_OK) return st;
    if (!d_info) return fail(SLA_ERR_INVALID_ARG, "NULL array");
    if (Ac->n_rows == 0) return empty_solve_info(batch, d_info, static_cast<hipStream_t>(stream));
    if ((!d_vals && Ac->nnz > 0) || !d_b || !d_x) return fail(SLA_ERR_INVALID_ARG, "NULL array");
    sla_csr* A = const_cast<sla_csr*>(Ac);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lk(A->mu);
    if (opts->flags & SLA_BICGSTAB)
        st = run_bicgstab(A, A->krp, A->col, A->cap, batch, d_vals, d_b, d_x, opts, d_info, s);
    else
        st = run_cg(A, A->krp, A->col, A->cap, A->band, A->band_cap, A->split, batch, d_vals, d_b, d_x, opts,
                    d_info, s);
    if (st == SLA_OK && !(opts->flags & SLA_FIXED_ITERS)) {
        hipError_t e = timing_collect();
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "timing collect: %s", hipGetErrorString(e));
    }
    return st;
}

}  // extern "C"

namespace {

// Scratch of the allocation-free solve (sla_solve_noalloc): one call's CG / Jacobi /
// BiCGStab workspace, in a static device array instead of memory from an allocator.
// Every GPU the library runs on holds its own copy until the process ends.  In host
// code the array's name is not a device address: each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// address is handed to kernels.
constexpr size_t kScratchBytes = size_t(SLA_NOALLOC_SCRATCH_MIB) << 20;
__device__ __align__(256) char scratch[kScratchBytes];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

sla_status scratch_of_device(int dev, char** out)
{
    if (dev < 0 || dev >= kScratchDevices)
        return fail(SLA_ERR_UNSUPPORTED, "the allocation-free solve supports device ordinals below %d",
                    kScratchDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<char*>(g_scratch_ptr[dev]);
    return SLA_OK;
}

}  // namespace

extern "C" {

sla_status sla_solve_noalloc(const sla_csr* Ac, int64_t batch, const double* d_vals, const double* d_b, double* d_x,
                             const sla_cg_opts* opts, sla_cg_info* d_info, void* stream)
{
    sla_status st = check_common(Ac, batch);
    if (st != SLA_OK) return st;
    if (Ac->n_rows != Ac->n_cols) return fail(SLA_ERR_UNSUPPORTED, "solve needs a square matrix");
    if ((st = check_opts(opts)) != SLA_OK) return st;
    if (!d_info) return fail(SLA_ERR_INVALID_ARG, "NULL array");
    if (Ac->n_rows == 0) return empty_solve_info(batch, d_info, static_cast<hipStream_t>(stream));
    if ((!d_vals && Ac->nnz > 0) || !d_b || !d_x) return fail(SLA_ERR_INVALID_ARG, "NULL array");
    char* base = nullptr;
    if ((st = scratch_of_device(Ac->device, &base)) != SLA_OK) return st;
    const FixedWs fx{base, kScratchBytes};
    sla_csr* A = const_cast<sla_csr*>(Ac);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lk(A->mu);
    if (opts->flags & SLA_BICGSTAB)
        st = run_bicgstab(A, A->krp, A->col, A->cap, batch, d_vals, d_b, d_x, opts, d_info, s, &fx);
    else
        st = run_cg(A, A->krp, A->col, A->cap, A->band, A->band_cap, A->split, batch, d_vals, d_b, d_x, opts,
                    d_info, s, nullptr, &fx);
    if (st == SLA_OK && !(opts->flags & SLA_FIXED_ITERS)) {
        hipError_t e = timing_collect();
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "timing collect: %s", hipGetErrorString(e));
    }
    return st;
}

sla_status sla_solve_backward(const sla_csr* Ac, int64_t batch, const double* d_vals, const double* d_x,
                              const double* d_gx, double* d_gb, double* d_gvals, const sla_cg_opts* opts,
                              sla_cg_info* d_info, void* stream)
{
    sla_status st = check_common(Ac, batch);
    if (st != SLA_OK) return st;
    if (Ac->n_rows != Ac->n_cols) return fail(SLA_ERR_UNSUPPORTED, "solve_backward needs a square matrix");
    if ((st = check_opts(opts)) != SLA_OK) return st;
    if (!d_info) return fail(SLA_ERR_INVALID_ARG, "NULL array");
    if (Ac->n_rows == 0) return empty_solve_info(batch, d_info, static_cast<hipStream_t>(stream));
    if ((!d_vals && Ac->nnz > 0) || !d_gx || !d_gb || (d_gvals && !d_x))
        return fail(SLA_ERR_INVALID_ARG, "NULL array");
    sla_csr* A = const_cast<sla_csr*>(Ac);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lk(A->mu);
    const bool bicg = (opts->flags & SLA_BICGSTAB) != 0;
    if (A->flags & SLA_SYMMETRIC) {
        st = bicg ? run_bicgstab(A, A->krp, A->col, A->cap, batch, d_vals, d_gx, d_gb, opts, d_info, s)
                  : run_cg(A, A->krp, A->col, A->cap, A->band, A->band_cap, A->split, batch, d_vals, d_gx, d_gb,
                           opts, d_info, s);
    } else {
        if ((st = ensure_transpose(A, s)) != SLA_OK) return st;
        const double* vt = nullptr;
        if ((st = ensure_vals_t(A, batch, d_vals, s, &vt)) != SLA_OK) return st;
        st = bicg ? run_bicgstab(A, A->row_ptr_t, A->col_t, A->cap_t, batch, vt, d_gx, d_gb, opts, d_info, s)
                  : run_cg(A, A->row_ptr_t, A->col_t, A->cap_t, 0, 0, A->split, batch, vt, d_gx, d_gb, opts,
                           d_info, s);
    }
    if (st != SLA_OK) return st;
    if (d_gvals) {
        hipError_t e = timed(SLA_K_PATTERN_OUTER, s, [&] {
            return launch_pattern_outer(A->krp, A->krp_bits, A->col, -1.0, d_gb, A->n_rows, d_x, A->n_cols,
                                        d_gvals, A->n_rows, A->nnz, static_cast<int>(batch), s);
        });
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "gradient scatter launch: %s", hipGetErrorString(e));
    }
    if (!(opts->flags & SLA_FIXED_ITERS)) {
        hipError_t e = timing_collect();
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "timing collect: %s", hipGetErrorString(e));
    }
    return SLA_OK;
}

sla_status sla_eigsh(const sla_csr* Ac, const double* d_vals, int32_t k, const double* d_v0, double* d_evals,
                     double* d_evecs, const sla_eig_opts* opts, sla_eig_info* info, void* stream)
{
    sla_status st = check_common(Ac, 1);
    if (st != SLA_OK) return st;
    if (Ac->n_rows != Ac->n_cols) return fail(SLA_ERR_UNSUPPORTED, "eigsh needs a square matrix");
    if (!(Ac->flags & SLA_SYMMETRIC))
        return fail(SLA_ERR_UNSUPPORTED, "eigsh needs a symmetric matrix (a handle created with SLA_SYMMETRIC)");
    if (!opts || !info || !d_v0 || !d_evals || !d_evecs || (!d_vals && Ac->nnz > 0))
        return fail(SLA_ERR_INVALID_ARG, "NULL argument");
    const int64_t n = Ac->n_rows;
    if (n < 1) return fail(SLA_ERR_INVALID_ARG, "eigsh of an empty matrix");
    const int64_t max_dim = opts->max_dim > 0 ? opts->max_dim : std::min<int64_t>(n, 1000);
    if (max_dim > n) return fail(SLA_ERR_INVALID_ARG, "max_dim %lld exceeds n %lld", (long long)max_dim, (long long)n);
    if (k < 1 || k > SLA_EIG_MAX_K || k > max_dim)
        return fail(SLA_ERR_INVALID_ARG, "k must be in [1, min(%d, max_dim)] (got %d)", SLA_EIG_MAX_K, k);
    if (!(opts->tol > 0.0)) return fail(SLA_ERR_INVALID_ARG, "tol must be > 0");
    if (opts->which != SLA_EIG_LARGEST && opts->which != SLA_EIG_SMALLEST)
        return fail(SLA_ERR_INVALID_ARG, "which must be SLA_EIG_LARGEST or SLA_EIG_SMALLEST");
    if (opts->check_every < 0) return fail(SLA_ERR_INVALID_ARG, "check_every must be >= 0");
    if (opts->max_iter < 0 || opts->keep < 0) return fail(SLA_ERR_INVALID_ARG, "max_iter and keep must be >= 0");
    if (opts->flags != 0) return fail(SLA_ERR_INVALID_ARG, "flags: the Lanczos eigensolver takes none");
    // thick restart when the step budget exceeds the basis size
    const int64_t total = std::max<int64_t>(max_dim, opts->max_iter);
    const bool restart = total > max_dim;
    const int64_t lk = opts->keep > 0 ? opts->keep
                                      : std::min<int64_t>(max_dim - 1, std::max<int64_t>(k + 1, (max_dim + k) / 2));
    if (restart) {
        static_assert(kEigRestartMaxDim == SLA_EIG_RESTART_MAX_DIM && kEigRestartMaxDim <= kLzStage, "caps");
        if (max_dim > kEigRestartMaxDim)
            return fail(SLA_ERR_INVALID_ARG, "thick restart needs max_dim <= %lld (got %lld)",
                        (long long)kEigRestartMaxDim, (long long)max_dim);
        if (lk < k || lk >= max_dim)
            return fail(SLA_ERR_INVALID_ARG, "thick restart needs k <= keep < max_dim (keep %lld)", (long long)lk);
    }
    const int64_t nS = restart ? std::max<int64_t>(k, lk) : k;   // Ritz coefficient rows
    sla_csr* A = const_cast<sla_csr*>(Ac);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> guard(A->mu);
    if ((st = ensure_col16(A, s)) != SLA_OK) return st;
    const bool largest = opts->which == SLA_EIG_LARGEST;
    const int rp_bits = A->krp_bits;
    const int64_t ntiles = (n + kTile - 1) / kTile;
    const int G = blocks_per_system(A, ntiles, 1, bs_blocks_per_cu(rp_bits, A->cap, n));
    const int Gu = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(1024, (n + kBlock - 1) / kBlock)));
    const int Gd = static_cast<int>((n + kLzRows - 1) / kLzRows);

    // device workspace
    const size_t sz_V = align256(sizeof(double) * static_cast<size_t>(max_dim + 1) * n);
    const size_t sz_w = align256(sizeof(double) * n);
    const size_t sz_ph = align256(sizeof(double) * static_cast<size_t>(max_dim + 1) * Gd);
    const size_t sz_md = align256(sizeof(double) * (max_dim + 1));
    const size_t sz_G = align256(sizeof(double) * G);
    const size_t sz_Gu = align256(sizeof(double) * Gu);
    const size_t sz_S = align256(sizeof(double) * static_cast<size_t>(nS) * max_dim);
    const size_t sz_k = align256(sizeof(double) * k);
    const size_t sz_pr = align256(sizeof(double) * 2 * k * Gu);
    const size_t need = sz_V + sz_w + sz_ph + 3 * sz_md + 2 * sz_G + sz_Gu + sz_S + sz_k + sz_pr +
                        align256(sizeof(SysState));
    if (need > A->eig_ws_bytes) {
        if (A->eig_ws) {
            HIP_TRY(hipDeviceSynchronize());
            HIP_TRY(dev_free(A->eig_ws));
            A->eig_ws = nullptr;
            A->eig_ws_bytes = 0;
        }
        if ((st = dev_alloc(&A->eig_ws, need)) != SLA_OK) return st;
        A->eig_ws_bytes = need;
    }
    // pinned host staging: alpha, beta, S, theta / scale, partials, restart couplings, state
    const size_t hneed = sizeof(double) * (2 * max_dim + static_cast<size_t>(nS) * max_dim + k + 2 * k * Gu + Gu +
                                           max_dim) +
                         sizeof(SysState);
    if (hneed > A->eig_host_bytes) {
        HIP_TRY(hipStreamSynchronize(s));
        if (A->eig_host) HIP_TRY(hipHostFree(A->eig_host));
        A->eig_host = nullptr;
        A->eig_host_bytes = 0;
        HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&A->eig_host), hneed, hipHostMallocDefault));
        A->eig_host_bytes = hneed;
    }
    char* p = static_cast<char*>(A->eig_ws);
    auto take = [&](size_t b) {
        char* q = p;
        p += b;
        return reinterpret_cast<double*>(q);
    };
    LzArgs a{};
    a.V = take(sz_V);
    a.w = take(sz_w);
    a.part_h = take(sz_ph);
    a.h = take(sz_md);
    a.alpha = take(sz_md);
    a.beta = take(sz_md);
    double* part_sigma = take(sz_G);
    double* part_tt = take(sz_G);
    a.part = take(sz_Gu);
    double* d_S = take(sz_S);
    double* d_scale = take(sz_k);
    a.part_ritz = take(sz_pr);
    SysState* d_st = reinterpret_cast<SysState*>(p);
    a.v0 = d_v0;
    a.part_sigma = part_sigma;
    a.S = d_S;
    a.U = d_evecs;
    a.scale = d_scale;
    a.n = n;
    a.G = G;
    a.Gu = Gu;
    a.Gd = Gd;
    a.k = k;
    double* h_ab = A->eig_host;                 // alpha [max_dim], beta [max_dim]
    double* h_S = h_ab + 2 * max_dim;           // [nS][m]
    double* h_theta = h_S + static_cast<size_t>(nS) * max_dim;
    double* h_part = h_theta + k;               // [2 k][Gu] (also the |v0|^2 partials)
    double* h_coup = h_part + 2 * k * Gu + Gu;  // [lk] couplings of the kept vectors
    SysState* h_st = reinterpret_cast<SysState*>(h_coup + max_dim);

    // the SpMV (BiCGStab's t = A s mode): operand v_j, product w, partials <v_j, w>
    CgArgs c{};
    c.row_ptr = A->krp;
    c.col = A->col;
    c.col16 = A->col16;
    c.vals = d_vals;
    c.z = a.w;
    c.part_sigma = part_sigma;
    c.part_tt = part_tt;
    c.st = d_st;
    c.n = n;
    c.nnz = A->nnz;
    c.ntiles = ntiles;
    c.G = G;
    c.Gu = Gu;
    c.batch = 1;
    c.xcd_remap = 1;
    c.split = 1;
    *h_st = SysState{};
    h_st->stop_iter = INT64_MAX;
    HIP_TRY(hipMemcpyAsync(d_st, h_st, sizeof(SysState), hipMemcpyHostToDevice, s));

    hipError_t e = timed(SLA_K_LZ_RITZ, s, [&] { return launch_lz(0, a, 0, 0.0, 0, s); });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "eigsh start: %s", hipGetErrorString(e));
    HIP_TRY(hipMemcpyAsync(h_part, a.part, sizeof(double) * Gu, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    double nn = 0.0;
    for (int g = 0; g < Gu; ++g) nn += h_part[g];
    const double nrm = std::sqrt(nn);
    if (!(nrm > 0.0) || !std::isfinite(nrm)) return fail(SLA_ERR_INVALID_ARG, "start vector v0 is zero or not finite");
    e = timed(SLA_K_LZ_RITZ, s, [&] { return launch_lz(1, a, 0, nrm, 0, s); });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "eigsh start: %s", hipGetErrorString(e));

    // Step j.  couple: the first step after a restart, which removes the couplings of the
    // kept vectors (staged in h) instead of beta_{j-1} v_{j-1} (beta[j-1] is 0 there).
    auto lanczos_step = [&](int64_t j, bool couple) -> hipError_t {
        c.p1 = a.V + j * n;
        hipError_t e0 = timed(SLA_K_LZ_SPMV, s, [&] { return launch_bs(4, c, j, rp_bits, A->cap, s); });
        if (e0 == hipSuccess) e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(2, a, j, 0.0, 0, s); });
        if (e0 == hipSuccess && couple) e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(5, a, j, 0.0, 0, s); });
        if (j + 1 <= kLzFusedCols) {
            // dots, reduce, (update + second dots), reduce, update with |w|^2 partials
            if (e0 == hipSuccess) e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(3, a, j + 1, 0.0, 0, s); });
            if (e0 == hipSuccess) e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(4, a, j + 1, 0.0, 0, s); });
            if (e0 == hipSuccess) e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz_axpy_dots(a, j + 1, s); });
            if (e0 == hipSuccess) e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(4, a, j + 1, 0.0, 0, s); });
            if (e0 == hipSuccess) e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(5, a, j + 1, 0.0, 1, s); });
        } else {
            for (int pass = 0; pass < 2 && e0 == hipSuccess; ++pass) {
                e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(3, a, j + 1, 0.0, 0, s); });
                if (e0 == hipSuccess) e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(4, a, j + 1, 0.0, 0, s); });
                if (e0 == hipSuccess)
                    e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(5, a, j + 1, 0.0, pass == 1, s); });
            }
        }
        if (e0 == hipSuccess) e0 = timed(SLA_K_LZ_ORTH, s, [&] { return launch_lz(6, a, j, 0.0, 0, s); });
        return e0;
    };

    const int64_t chunk = opts->check_every > 0 ? opts->check_every : 16;
    // beta_j at the rounding level of the reorthogonalized w (<= sqrt(n) eps |T|, |T| the
    // largest row sum of the projected matrix with beta_j) means the Krylov space is
    // numerically invariant
    const double inv_level = std::sqrt(static_cast<double>(n)) * DBL_EPSILON;
    double tnorm = 0.0;
    int64_t j = 0, m_stop = -1, steps = 0, jcouple = -1;
    int32_t restarts = 0;
    int state = SLA_MAX_ITER;
    double max_res = 0.0;
    std::vector<double> theta(nS), res(k);
    // restart mode: the projected matrix of the current basis, [(max_dim + 1)]^2 row-major
    // (tridiagonal until the first restart, then diag(theta) bordered by the couplings)
    const int64_t ld = max_dim + 1;
    std::vector<double> H, Hm;
    if (restart) {
        H.assign(static_cast<size_t>(ld) * ld, 0.0);
        Hm.resize(static_cast<size_t>(max_dim) * max_dim);
    }
    auto Hat = [&](int64_t r, int64_t q) -> double& { return H[static_cast<size_t>(r) * ld + q]; };
    while (m_stop < 0) {
        const int64_t j0 = j;
        int64_t jend = std::min<int64_t>(j + chunk, max_dim);
        if (restart) jend = std::min<int64_t>(jend, j + (total - steps));
        for (; j < jend; ++j) {
            if ((e = lanczos_step(j, j == jcouple)) != hipSuccess)
                return fail(SLA_ERR_HIP, "eigsh step: %s", hipGetErrorString(e));
        }
        HIP_TRY(hipMemcpyAsync(h_ab + j0, a.alpha + j0, sizeof(double) * (jend - j0), hipMemcpyDeviceToHost, s));
        HIP_TRY(hipMemcpyAsync(h_ab + max_dim + j0, a.beta + j0, sizeof(double) * (jend - j0), hipMemcpyDeviceToHost,
                               s));
        HIP_TRY(hipStreamSynchronize(s));
        const double* al = h_ab;
        const double* be = h_ab + max_dim;
        for (int64_t jj = j0; jj < jend && m_stop < 0; ++jj) {
            const int64_t m = jj + 1;
            ++steps;
            double b = be[jj];
            if (!restart) {
                tnorm = std::max(tnorm, std::fabs(al[jj]) + std::fabs(b) + (jj > 0 ? std::fabs(be[jj - 1]) : 0.0));
                if (b <= inv_level * tnorm) b = 0.0;
                if (m < k) {
                    if (b == 0.0) {
                        m_stop = m;
                        state = SLA_BREAKDOWN;
                    }
                    continue;
                }
                tridiag_eigpairs(al, be, static_cast<int>(m), k, largest, theta.data(), h_S);
            } else {
                Hat(jj, jj) = al[jj];
                Hat(jj, jj + 1) = Hat(jj + 1, jj) = b;
                double row = 0.0;   // rows above jj keep their sums
                for (int64_t q = 0; q <= m; ++q) row += std::fabs(Hat(jj, q));
                tnorm = std::max(tnorm, row);
                if (b <= inv_level * tnorm) {
                    b = 0.0;
                    Hat(jj, jj + 1) = Hat(jj + 1, jj) = 0.0;
                }
                if (!(m == max_dim || b == 0.0 || steps == total)) continue;
                if (m < k) {   // invariant before k Ritz values exist
                    m_stop = m;
                    state = SLA_BREAKDOWN;
                    continue;
                }
                for (int64_t r = 0; r < m; ++r)
                    std::copy(&Hat(r, 0), &Hat(r, 0) + m, Hm.begin() + static_cast<size_t>(r) * m);
                const bool may_restart = m == max_dim && b != 0.0 && steps < total;
                sym_eigpairs(Hm.data(), static_cast<int>(m), static_cast<int>(may_restart ? lk : k), largest,
                             theta.data(), h_S);
            }
            bool done = true;
            max_res = 0.0;
            for (int r = 0; r < k; ++r) {
                res[r] = b * std::fabs(h_S[static_cast<size_t>(r) * m + m - 1]);
                max_res = std::max(max_res, res[r]);
                if (!(res[r] <= opts->tol * std::fabs(theta[r]))) done = false;
            }
            if (done || b == 0.0) {
                m_stop = m;
                state = SLA_CONVERGED;
            } else if (!restart ? m == max_dim : steps == total) {
                m_stop = m;
                state = SLA_MAX_ITER;
            } else if (restart && m == max_dim) {
                // thick restart: the lk wanted-end Ritz vectors V S^T, then v_m, start the
                // new basis; the projected matrix becomes diag(theta) bordered by the
                // couplings beta s_r[m-1] (Wu and Simon 2000)
                a.m = m;
                HIP_TRY(hipMemcpyAsync(d_S, h_S, sizeof(double) * lk * m, hipMemcpyHostToDevice, s));
                e = timed(SLA_K_LZ_RITZ, s, [&] { return launch_lz_restart(a, m, lk, s); });
                if (e != hipSuccess) return fail(SLA_ERR_HIP, "eigsh restart: %s", hipGetErrorString(e));
                std::fill(H.begin(), H.end(), 0.0);
                tnorm = 0.0;
                for (int64_t r = 0; r < lk; ++r) {
                    const double cr = b * h_S[static_cast<size_t>(r) * m + m - 1];
                    Hat(r, r) = theta[r];
                    Hat(r, lk) = Hat(lk, r) = cr;
                    h_coup[r] = cr;
                    tnorm = std::max(tnorm, std::fabs(theta[r]) + std::fabs(cr));
                }
                // the first step of the new basis subtracts sum_r c_r v_r through h, and
                // no beta_{lk-1} v_{lk-1}
                HIP_TRY(hipMemcpyAsync(a.h, h_coup, sizeof(double) * lk, hipMemcpyHostToDevice, s));
                HIP_TRY(hipMemsetAsync(a.beta + (lk - 1), 0, sizeof(double), s));
                j = jcouple = lk;
                ++restarts;
            }
        }
    }
    info->iterations = steps;
    info->state = state;
    info->restarts = restarts;
    if (state == SLA_BREAKDOWN) {
        info->max_res = 0.0;
        return SLA_OK;   // d_evals / d_evecs untouched: fewer than k Ritz values exist
    }
    info->max_res = max_res;
    // Ritz vectors of the stopping step: u_r = V_m s_r, then divided by their signed norms
    a.m = m_stop;
    HIP_TRY(hipMemcpyAsync(d_S, h_S, sizeof(double) * k * m_stop, hipMemcpyHostToDevice, s));
    e = timed(SLA_K_LZ_RITZ, s, [&] { return launch_lz(7, a, 0, 0.0, 0, s); });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "eigsh ritz: %s", hipGetErrorString(e));
    HIP_TRY(hipMemcpyAsync(h_part, a.part_ritz, sizeof(double) * 2 * k * Gu, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    for (int r = 0; r < k; ++r) {
        double uu = 0.0, uv = 0.0;
        for (int g = 0; g < Gu; ++g) {
            uu += h_part[static_cast<size_t>(2 * r) * Gu + g];
            uv += h_part[static_cast<size_t>(2 * r + 1) * Gu + g];
        }
        const double nu = std::sqrt(uu);
        h_theta[r] = uv < 0.0 ? -nu : nu;   // staged as the signed norms first
    }
    HIP_TRY(hipMemcpyAsync(d_scale, h_theta, sizeof(double) * k, hipMemcpyHostToDevice, s));
    e = timed(SLA_K_LZ_RITZ, s, [&] { return launch_lz(8, a, 0, 0.0, 0, s); });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "eigsh scale: %s", hipGetErrorString(e));
    HIP_TRY(hipStreamSynchronize(s));
    for (int r = 0; r < k; ++r) h_theta[r] = theta[r];
    HIP_TRY(hipMemcpyAsync(d_evals, h_theta, sizeof(double) * k, hipMemcpyHostToDevice, s));
    HIP_TRY(hipStreamSynchronize(s));
    hipError_t te = timing_collect();
    if (te != hipSuccess) return fail(SLA_ERR_HIP, "timing collect: %s", hipGetErrorString(te));
    return SLA_OK;
}

}  // extern "C"

namespace {

// Cholesky G = L L^T of the symmetrized m x m G (row-major) with the pivot test of the
// block orthonormalization (every pivot above kOrthPivot times the largest diagonal
// entry); on success Rinv = (L^T)^-1, upper triangular, by back substitution.
constexpr double kOrthPivot = 1e-14;
bool chol_rinv(const std::vector<double>& G0, int m, std::vector<double>& Rinv)
{
    std::vector<double> G(static_cast<size_t>(m) * m), L(static_cast<size_t>(m) * m, 0.0);
    double gmax = 0.0;
    for (int a = 0; a < m; ++a)
        for (int b = 0; b < m; ++b) G[a * m + b] = 0.5 * (G0[a * m + b] + G0[b * m + a]);
    for (int a = 0; a < m; ++a) gmax = std::max(gmax, G[a * m + a]);
    for (int j = 0; j < m; ++j) {
        double d = G[j * m + j];
        for (int p = 0; p < j; ++p) d -= L[j * m + p] * L[j * m + p];
        if (!(d > kOrthPivot * gmax)) return false;
        L[j * m + j] = std::sqrt(d);
        for (int i = j + 1; i < m; ++i) {
            double t = G[i * m + j];
            for (int p = 0; p < j; ++p) t -= L[i * m + p] * L[j * m + p];
            L[i * m + j] = t / L[j * m + j];
        }
    }
    // R = L^T upper; solve R X = I column by column
    Rinv.assign(static_cast<size_t>(m) * m, 0.0);
    for (int c = 0; c < m; ++c)
        for (int i = c; i >= 0; --i) {
            double t = (i == c) ? 1.0 : 0.0;
            for (int p = i + 1; p <= c; ++p) t -= L[p * m + i] * Rinv[p * m + c];
            Rinv[i * m + c] = t / L[i * m + i];
        }
    return true;
}

// Device-side staging of the small per-launch arrays (index lists, coefficient
// matrices): appended to a pinned arena, then one copy in stream order per launch
// (flush) for everything appended since the last; the arena is reset only after the
// host has synchronized with the stream.
struct Arena {
    char* h = nullptr;
    char* d = nullptr;
    size_t cap = 0, off = 0, sent = 0;
    template <class T>
    const T* put(const T* src, size_t count, hipError_t& e)
    {
        const size_t bytes = sizeof(T) * count;
        if (off + bytes > cap) {
            e = hipErrorOutOfMemory;
            return nullptr;
        }
        std::memcpy(h + off, src, bytes);
        T* dst = reinterpret_cast<T*>(d + off);
        off = (off + bytes + 255) & ~static_cast<size_t>(255);
        e = hipSuccess;
        return dst;
    }
    hipError_t flush(hipStream_t s)
    {
        hipError_t e = hipSuccess;
        if (off > sent) e = hipMemcpyAsync(d + sent, h + sent, off - sent, hipMemcpyHostToDevice, s);
        sent = off;
        return e;
    }
    void reset() { off = sent = 0; }
};

}  // namespace

extern "C" {

sla_status sla_lobpcg(const sla_csr* Ac, const double* d_vals, int32_t k, const double* d_X0, double* d_evals,
                      double* d_evecs, const sla_eig_opts* opts, sla_eig_info* info, void* stream)
{
    sla_status st = check_common(Ac, 1);
    if (st != SLA_OK) return st;
    if (Ac->n_rows != Ac->n_cols) return fail(SLA_ERR_UNSUPPORTED, "lobpcg needs a square matrix");
    if (!(Ac->flags & SLA_SYMMETRIC))
        return fail(SLA_ERR_UNSUPPORTED, "lobpcg needs a symmetric matrix (a handle created with SLA_SYMMETRIC)");
    if (!opts || !info || !d_X0 || !d_evals || !d_evecs || (!d_vals && Ac->nnz > 0))
        return fail(SLA_ERR_INVALID_ARG, "NULL argument");
    const int64_t n = Ac->n_rows;
    if (k < 1 || k > SLA_EIG_MAX_K || 3 * static_cast<int64_t>(k) > n)
        return fail(SLA_ERR_INVALID_ARG, "k must be in [1, %d] with 3 k <= n (got k %d, n %lld)", SLA_EIG_MAX_K, k,
                    (long long)n);
    if (!(opts->tol > 0.0)) return fail(SLA_ERR_INVALID_ARG, "tol must be > 0");
    if (opts->which != SLA_EIG_LARGEST && opts->which != SLA_EIG_SMALLEST)
        return fail(SLA_ERR_INVALID_ARG, "which must be SLA_EIG_LARGEST or SLA_EIG_SMALLEST");
    if (opts->max_iter < 0) return fail(SLA_ERR_INVALID_ARG, "max_iter must be >= 0");
    if (opts->flags & ~SLA_EIG_JACOBI) return fail(SLA_ERR_INVALID_ARG, "unknown flags 0x%x", opts->flags);
    const bool jacobi = (opts->flags & SLA_EIG_JACOBI) != 0;
    static_assert(3 * SLA_EIG_MAX_K <= kBlkMaxCols, "block width");
    const int64_t max_iter = opts->max_iter > 0 ? opts->max_iter : 1000;
    const bool largest = opts->which == SLA_EIG_LARGEST;
    sla_csr* A = const_cast<sla_csr*>(Ac);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> guard(A->mu);

    // The block columns sit in fixed slots of k columns; the Ritz step's outputs (X, AX,
    // P, AP) alternate between two slots, so an iteration's index lists change only with
    // its active set.  The last column holds the Jacobi reciprocals.
    enum { kSX = 0, kSAX = 2, kSP = 4, kSAP = 6, kSR = 8, kSWa, kSWb, kSWc, kSAW, kSPa, kSPb, kSAPa, kSAPb, kSlots };
    const int NC = kSlots * k + 1;
    const int Gg = blk_gram_groups(n), Gc = blk_comb_groups(n);
    const size_t kk9 = 9 * static_cast<size_t>(k) * k;
    constexpr size_t kListCap = 1 << 16;   // int32 entries of the device list table
    const size_t sz_pool = align256(sizeof(double) * static_cast<size_t>(NC) * n);
    const size_t sz_gp = align256(sizeof(double) * static_cast<size_t>(Gg) * kk9);
    const size_t sz_sm = align256(sizeof(double) * kk9);
    const size_t sz_cp = align256(sizeof(double) * static_cast<size_t>(Gc) * k);
    const size_t sz_lists = align256(sizeof(int32_t) * kListCap);
    const size_t sz_arena = 1 << 20;
    const size_t need = sz_pool + sz_gp + 2 * sz_sm + sz_cp + sz_lists + sz_arena;
    if (need > A->lob_ws_bytes) {
        if (A->lob_ws) {
            HIP_TRY(hipDeviceSynchronize());
            HIP_TRY(dev_free(A->lob_ws));
            A->lob_ws = nullptr;
            A->lob_ws_bytes = 0;
        }
        if ((st = dev_alloc(&A->lob_ws, need)) != SLA_OK) return st;
        A->lob_ws_bytes = need;
    }
    const size_t hneed = sz_arena + sz_lists;
    if (hneed > A->lob_host_bytes) {
        HIP_TRY(hipStreamSynchronize(s));
        if (A->lob_host) HIP_TRY(hipHostFree(A->lob_host));
        A->lob_host = nullptr;
        A->lob_host_bytes = 0;
        HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&A->lob_host), hneed, hipHostMallocDefault));
        A->lob_host_bytes = hneed;
    }
    // results the kernels write straight into host memory (coherent, so a stream
    // synchronization is all the host waits for): a Gram matrix, the squared residual
    // norms, the W and P block flags
    const size_t rneed = sizeof(double) * (kk9 + k + 2);
    if (rneed > A->lob_res_bytes) {
        HIP_TRY(hipStreamSynchronize(s));
        if (A->lob_res) HIP_TRY(hipHostFree(A->lob_res));
        A->lob_res = nullptr;
        A->lob_res_bytes = 0;
        HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&A->lob_res), rneed, hipHostMallocCoherent));
        A->lob_res_bytes = rneed;
    }
    double* hH = A->lob_res;
    double* hN = hH + kk9;
    double* hF = hN + k;
    double* dH = nullptr;
    HIP_TRY(hipHostGetDevicePointer(reinterpret_cast<void**>(&dH), A->lob_res, 0));
    double* dN = dH + kk9;
    double* dF = dN + k;

    char* p = static_cast<char*>(A->lob_ws);
    double* pool = reinterpret_cast<double*>(p);
    p += sz_pool;
    double* d_gpart = reinterpret_cast<double*>(p);
    p += sz_gp;
    double* d_cg = reinterpret_cast<double*>(p);   // Gram matrices the device factors
    p += sz_sm;
    double* d_cy = reinterpret_cast<double*>(p);   // coefficient matrices formed on the device
    p += sz_sm;
    double* d_cpart = reinterpret_cast<double*>(p);
    p += sz_cp;
    int32_t* d_lists = reinterpret_cast<int32_t*>(p);
    p += sz_lists;
    Arena ar;   // per-step uploads: the Ritz and residual coefficients
    ar.d = p;
    ar.h = A->lob_host;
    ar.cap = sz_arena;
    double* tinv = pool + static_cast<size_t>(NC - 1) * n;

    // Index lists, uploaded once and kept on the device while the active set lasts.
    // get() stages a new list on the host; flush() sends what is staged in one copy.
    // Tables fill only after a synchronization, so a reset never pulls a list from
    // under a kernel in flight.
    struct Lists {
        int32_t* h = nullptr;
        int32_t* d = nullptr;
        size_t off = 0, sent = 0;
        std::map<std::vector<int32_t>, size_t> at;
        const int32_t* get(const std::vector<int32_t>& v)
        {
            auto it = at.find(v);
            if (it != at.end()) return d + it->second;
            std::memcpy(h + off, v.data(), sizeof(int32_t) * v.size());
            at.emplace(v, off);
            const int32_t* q = d + off;
            off += v.size();
            return q;
        }
        void room(size_t need)
        {
            if (off + need > kListCap) {
                at.clear();
                off = sent = 0;
            }
        }
        hipError_t flush(hipStream_t st)
        {
            hipError_t e = hipSuccess;
            if (off > sent)
                e = hipMemcpyAsync(d + sent, h + sent, sizeof(int32_t) * (off - sent), hipMemcpyHostToDevice, st);
            sent = off;
            return e;
        }
    } lists;
    lists.h = reinterpret_cast<int32_t*>(A->lob_host + sz_arena);
    lists.d = d_lists;
    const size_t kPhaseLists = 64 * static_cast<size_t>(kBlkMaxCols);   // more than one step's lists

    using Cols = std::vector<int32_t>;
    auto slot = [&](int sl, const std::vector<int>& idx) {
        Cols c(idx.size());
        for (size_t i = 0; i < idx.size(); ++i) c[i] = sl * k + idx[i];
        return c;
    };
    auto cat = [](std::initializer_list<const Cols*> parts) {
        Cols o;
        for (const Cols* q : parts) o.insert(o.end(), q->begin(), q->end());
        return o;
    };
    std::vector<int> allk(k);
    for (int r = 0; r < k; ++r) allk[r] = r;
    hipError_t e = hipSuccess;
    auto hip_fail = [&](const char* what) { return fail(SLA_ERR_HIP, "lobpcg %s: %s", what, hipGetErrorString(e)); };
    const bool even = (n % 2) == 0;
    auto aligned = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };

    // launches on column lists already on the device
    auto gram = [&](const double* ba, const int32_t* la, int mu, const double* bb, const int32_t* lb, int mv,
                    bool same, double* out, double* yproj = nullptr) -> hipError_t {
        return timed(SLA_K_LOB_GRAM, s, [&] {
            return launch_blk_gram(ba, la, mu, bb, lb, mv, n, d_gpart, out, s, same, yproj);
        }, false, 8.0 * static_cast<double>(n) * (same ? mu : mu + mv));
    };
    auto comb = [&](const double* bin, const int32_t* lin, int m, const double* dY, double* bout,
                    const int32_t* lout, int q, double* norms) -> hipError_t {
        hipError_t r = timed(SLA_K_LOB_COMB, s, [&] {
            // pairs of rows with 16-byte accesses where every column base allows it
            const bool pairs = even && aligned(bin) && aligned(bout);
            return launch_blk_comb(bin, lin, m, dY, bout, lout, q, n, norms ? d_cpart : nullptr, s, pairs);
        }, true, 8.0 * static_cast<double>(n) * (m + q));
        if (r == hipSuccess && norms)
            r = timed(SLA_K_LOB_COMB, s, [&] { return launch_blk_reduce(d_cpart, Gc, q, norms, s); });
        return r;
    };
    auto spmm = [&](const int32_t* lin, const int32_t* lout, int q) -> hipError_t {
        // values, columns and row pointers once, each input column once (the gathers are
        // cache traffic), each output column written
        const double bytes = 12.0 * static_cast<double>(A->nnz) + (A->krp_bits / 8.0) * static_cast<double>(n + 1) +
                             16.0 * static_cast<double>(n) * static_cast<double>(q);
        return timed(SLA_K_LOB_SPMM, s, [&] {
            return launch_blk_spmm(A->krp, A->krp_bits, A->col, d_vals, pool, lin, pool, lout, q, n, s);
        }, true, bytes);
    };
    // the Cholesky QR coefficients of a block (its Gram and factorization) into d_cy
    auto orth_coef = [&](const double* bz, const int32_t* lz, int w, bool scale, double* flag) -> hipError_t {
        return timed(SLA_K_LOB_GRAM, s, [&] {
            return launch_blk_gram_orth(bz, lz, w, n, d_gpart, d_cg, scale, kOrthPivot, flag, d_cy, s);
        }, false, 8.0 * static_cast<double>(n) * w);
    };
    // Z (w columns; AZ alike when given) out of place through two Cholesky QR passes,
    // unit-scaled first, ending in slots z2 (and az2); flag: the block's flag
    auto orth = [&](const double* bz, const int32_t* lz, const int32_t* lz1, const int32_t* lz2,
                    const int32_t* laz, const int32_t* laz1, const int32_t* laz2, int w, double* flag) -> hipError_t {
        // pass 0: Z -> Z1 (AZ -> AZ1), pass 1: Z1 -> Z2 (AZ1 -> AZ2)
        if ((e = orth_coef(bz, lz, w, true, flag)) != hipSuccess) return e;
        if ((e = comb(bz, lz, w, d_cy, pool, lz1, w, nullptr)) != hipSuccess) return e;
        if (laz && (e = comb(pool, laz, w, d_cy, pool, laz1, w, nullptr)) != hipSuccess) return e;
        if ((e = orth_coef(pool, lz1, w, false, flag)) != hipSuccess) return e;
        if ((e = comb(pool, lz1, w, d_cy, pool, lz2, w, nullptr)) != hipSuccess) return e;
        if (laz && (e = comb(pool, laz1, w, d_cy, pool, laz2, w, nullptr)) != hipSuccess) return e;
        return hipSuccess;
    };
    // one projection pass Z - B (B^T Z) (AZ - AB (B^T Z)) into slots z1 (az1); lzb lists
    // [Z, B], lazb [AZ, AB]
    auto project = [&](const int32_t* lb, int b, const int32_t* lz, const int32_t* lzb, const int32_t* lz1,
                       const int32_t* lazb, const int32_t* laz1, int w) -> hipError_t {
        // C = B^T Z [b][w], written as the coefficients [I; -C] over [Z, B]
        if ((e = gram(pool, lb, b, pool, lz, w, false, nullptr, d_cy)) != hipSuccess) return e;
        if ((e = comb(pool, lzb, w + b, d_cy, pool, lz1, w, nullptr)) != hipSuccess) return e;
        if (lazb && (e = comb(pool, lazb, w + b, d_cy, pool, laz1, w, nullptr)) != hipSuccess) return e;
        return hipSuccess;
    };
    // Rayleigh-Ritz on the orthonormal S of m columns (H = S^T AS in hH), keeping the
    // columns listed: theta (k), Y [m][k] with zero rows for the columns left out, and
    // the residual coefficients Yr [2k][k] = [I; -diag(theta)]; both uploaded
    std::vector<double> theta(k), Y, Yr;
    const double *dY = nullptr, *dYr = nullptr;
    auto rayleigh_ritz = [&](int m, const std::vector<int>& keep) -> hipError_t {
        const int me = static_cast<int>(keep.size());
        std::vector<double> Hs(static_cast<size_t>(me) * me), Ys(static_cast<size_t>(k) * me);
        for (int a = 0; a < me; ++a)
            for (int b = 0; b < me; ++b)
                Hs[a * me + b] = 0.5 * (hH[keep[a] * m + keep[b]] + hH[keep[b] * m + keep[a]]);
        sym_eigpairs(Hs.data(), me, k, largest, theta.data(), Ys.data());
        Y.assign(static_cast<size_t>(m) * k, 0.0);
        for (int r = 0; r < k; ++r)
            for (int j = 0; j < me; ++j) Y[static_cast<size_t>(keep[j]) * k + r] = Ys[static_cast<size_t>(r) * me + j];
        Yr.assign(static_cast<size_t>(2 * k) * k, 0.0);
        for (int r = 0; r < k; ++r) {
            Yr[r * k + r] = 1.0;
            Yr[(k + r) * k + r] = -theta[r];
        }
        ar.reset();
        dY = ar.put(Y.data(), Y.size(), e);
        if (e != hipSuccess) return e;
        dYr = ar.put(Yr.data(), Yr.size(), e);
        if (e != hipSuccess) return e;
        return ar.flush(s);
    };

    if (jacobi) {   // T = diag(A)^-1, with a count of the rows that have no usable a_ii
        e = timed(SLA_K_LOB_COMB, s, [&] {
            return launch_blk_diag_inv(A->krp, A->krp_bits, A->col, d_vals, n, tinv, d_cpart, s);
        });
        if (e == hipSuccess) e = timed(SLA_K_LOB_COMB, s, [&] { return launch_blk_reduce(d_cpart, Gc, 1, dN, s); });
        if (e != hipSuccess) return hip_fail("jacobi");
        HIP_TRY(hipStreamSynchronize(s));
        if (hN[0] != 0.0)
            return fail(SLA_ERR_INVALID_ARG, "Jacobi needs every diagonal entry stored, finite and positive (%.0f rows "
                        "have none)", hN[0]);
    }

    // start: X = orth(X0) into slot X[0], AX = A X, Rayleigh-Ritz on X, X = X Y into X[1]
    const Cols c_x0(allk.begin(), allk.end());   // the caller's rows of X0
    const Cols c_x[2] = {slot(kSX, allk), slot(kSX + 1, allk)}, c_ax[2] = {slot(kSAX, allk), slot(kSAX + 1, allk)};
    const Cols c_p[2] = {slot(kSP, allk), slot(kSP + 1, allk)}, c_ap[2] = {slot(kSAP, allk), slot(kSAP + 1, allk)};
    const Cols c_r = slot(kSR, allk), c_wa = slot(kSWa, allk);
    {
        lists.room(kPhaseLists);
        const int32_t* l_x0 = lists.get(c_x0);
        const int32_t* l_wa = lists.get(c_wa);
        const int32_t* l_x = lists.get(c_x[0]);
        const int32_t* l_ax = lists.get(c_ax[0]);
        const int32_t* l_x1 = lists.get(c_x[1]);
        const int32_t* l_ax1 = lists.get(c_ax[1]);
        if ((e = lists.flush(s)) != hipSuccess) return hip_fail("start");
        if ((e = orth(d_X0, l_x0, l_wa, l_x, nullptr, nullptr, nullptr, k, dF)) != hipSuccess) return hip_fail("start");
        HIP_TRY(hipStreamSynchronize(s));
        if (hF[0] == 0.0) return fail(SLA_ERR_INVALID_ARG, "start block X0 is rank deficient (or has a zero row)");
        if ((e = spmm(l_x, l_ax, k)) != hipSuccess) return hip_fail("start");
        if ((e = gram(pool, l_x, k, pool, l_ax, k, false, dH)) != hipSuccess) return hip_fail("start");
        HIP_TRY(hipStreamSynchronize(s));
        if ((e = rayleigh_ritz(k, allk)) != hipSuccess) return hip_fail("start");
        if ((e = comb(pool, l_x, k, dY, pool, l_x1, k, nullptr)) != hipSuccess) return hip_fail("start");
        if ((e = comb(pool, l_ax, k, dY, pool, l_ax1, k, nullptr)) != hipSuccess) return hip_fail("start");
    }
    int par = 1;         // X, AX (and P, AP) live in slot kSX + par ...
    bool has_p = false;  // no P before the first iteration
    int64_t it = 0;
    int state = SLA_MAX_ITER;
    std::vector<double> res(k);
    while (true) {
        // residuals R = A X - X diag(theta), their squared norms straight to host memory
        {
            const Cols in = cat({&c_ax[par], &c_x[par]});
            lists.room(kPhaseLists);
            const int32_t* l_in = lists.get(in);
            const int32_t* l_r = lists.get(c_r);
            if ((e = lists.flush(s)) != hipSuccess) return hip_fail("residual");
            if ((e = comb(pool, l_in, 2 * k, dYr, pool, l_r, k, dN)) != hipSuccess) return hip_fail("residual");
            HIP_TRY(hipStreamSynchronize(s));
        }
        std::vector<int> active;
        for (int r = 0; r < k; ++r) {
            res[r] = std::sqrt(hN[r]);
            if (res[r] > opts->tol * std::fabs(theta[r])) active.push_back(r);
        }
        if (active.empty() || it == max_iter) {
            state = active.empty() ? SLA_CONVERGED : SLA_MAX_ITER;
            break;
        }
        ++it;
        const int a = static_cast<int>(active.size());
        std::vector<int> ia(a);
        for (int j = 0; j < a; ++j) ia[j] = j;
        const Cols &X = c_x[par], &AX = c_ax[par];
        const Cols RA = slot(kSR, active), PA = slot(kSP + par, active), APA = slot(kSAP + par, active);
        const Cols Wa = slot(kSWa, ia), Wb = slot(kSWb, ia), Wc = slot(kSWc, ia), AW = slot(kSAW, ia);
        const Cols Pa = slot(kSPa, ia), Pb = slot(kSPb, ia), APa = slot(kSAPa, ia), APb = slot(kSAPb, ia);
        const Cols& Z0 = jacobi ? Wc : RA;
        const Cols Z0X = cat({&Z0, &X}), WaX = cat({&Wa, &X});
        const Cols B = cat({&X, &Wb}), AB = cat({&AX, &AW});
        const Cols PAB = cat({&PA, &B}), APAAB = cat({&APA, &AB}), PaB = cat({&Pa, &B}), APaAB = cat({&APa, &AB});
        const Cols S = has_p ? cat({&X, &Wb, &Pb}) : cat({&X, &Wb});
        const Cols AS = has_p ? cat({&AX, &AW, &APb}) : cat({&AX, &AW});
        const Cols Sk(S.begin() + k, S.end()), ASk(AS.begin() + k, AS.end());
        const int m = static_cast<int>(S.size());
        const int nx = 1 - par;
        lists.room(kPhaseLists);
        const int32_t *l_x = lists.get(X), *l_ra = lists.get(RA), *l_wc = lists.get(Wc), *l_z0 = lists.get(Z0);
        const int32_t *l_z0x = lists.get(Z0X), *l_wa = lists.get(Wa), *l_wax = lists.get(WaX), *l_wb = lists.get(Wb);
        const int32_t *l_aw = lists.get(AW), *l_s = lists.get(S), *l_as = lists.get(AS);
        const int32_t *l_sk = lists.get(Sk), *l_ask = lists.get(ASk);
        const int32_t *l_xn = lists.get(c_x[nx]), *l_axn = lists.get(c_ax[nx]);
        const int32_t *l_pn = lists.get(c_p[nx]), *l_apn = lists.get(c_ap[nx]);
        const int32_t *l_b = nullptr, *l_pa0 = nullptr, *l_pab = nullptr, *l_apab = nullptr, *l_pa = nullptr;
        const int32_t *l_apa = nullptr, *l_pa_b = nullptr, *l_apa_ab = nullptr, *l_pb = nullptr, *l_apb = nullptr;
        if (has_p) {
            l_b = lists.get(B);
            l_pa0 = lists.get(PA);
            l_pab = lists.get(PAB);
            l_apab = lists.get(APAAB);
            l_pa = lists.get(Pa);
            l_apa = lists.get(APa);
            l_pa_b = lists.get(PaB);
            l_apa_ab = lists.get(APaAB);
            l_pb = lists.get(Pb);
            l_apb = lists.get(APb);
        }
        if ((e = lists.flush(s)) != hipSuccess) return hip_fail("lists");
        // W = T R[:, active] with Jacobi, then made orthonormal against X and orthonormal
        if (jacobi) {
            e = timed(SLA_K_LOB_COMB, s, [&] { return launch_blk_rowscale(pool, l_ra, pool, l_wc, a, n, tinv, s); },
                      true, 8.0 * static_cast<double>(n) * (2 * a + 1));
            if (e != hipSuccess) return hip_fail("preconditioner");
        }
        if ((e = project(l_x, k, l_z0, l_z0x, l_wa, nullptr, nullptr, a)) != hipSuccess) return hip_fail("projection");
        if ((e = project(l_x, k, l_wa, l_wax, l_wb, nullptr, nullptr, a)) != hipSuccess) return hip_fail("projection");
        if ((e = orth(pool, l_wb, l_wa, l_wb, nullptr, nullptr, nullptr, a, dF)) != hipSuccess)
            return hip_fail("orthonormalization");
        if ((e = spmm(l_wb, l_aw, a)) != hipSuccess) return hip_fail("spmm");
        // P = P[:, active] (AP alike) made orthonormal against [X, W] and orthonormal; a
        // block that fails is zero from there on and left out of the Rayleigh-Ritz step
        if (has_p) {
            if ((e = project(l_b, k + a, l_pa0, l_pab, l_pa, l_apab, l_apa, a)) != hipSuccess)
                return hip_fail("projection");
            if ((e = project(l_b, k + a, l_pa, l_pa_b, l_pb, l_apa_ab, l_apb, a)) != hipSuccess)
                return hip_fail("projection");
            if ((e = orth(pool, l_pb, l_pa, l_pb, l_apb, l_apa, l_apb, a, dF + 1)) != hipSuccess)
                return hip_fail("orthonormalization");
        }
        if ((e = gram(pool, l_s, m, pool, l_as, m, false, dH)) != hipSuccess) return hip_fail("rayleigh-ritz");
        HIP_TRY(hipStreamSynchronize(s));
        std::vector<int> keep(allk);
        if (hF[0] != 0.0)
            for (int j = 0; j < a; ++j) keep.push_back(k + j);
        if (has_p && hF[1] != 0.0)
            for (int j = 0; j < a; ++j) keep.push_back(k + a + j);
        if ((e = rayleigh_ritz(m, keep)) != hipSuccess) return hip_fail("rayleigh-ritz");
        // X = S Y, AX = AS Y; P = S[k:] Y[k:], AP = AS[k:] Y[k:] (Knyazev's direction),
        // X and P in one pass over S (AX and AP over AS) where rows pair up
        if (even) {
            const double bytes = 8.0 * static_cast<double>(n) * (m + 2 * k);
            e = timed(SLA_K_LOB_COMB, s, [&] {
                return launch_blk_comb_dual(pool, l_s, m, k, dY, pool, l_xn, l_pn, k, n, s);
            }, true, bytes);
            if (e == hipSuccess)
                e = timed(SLA_K_LOB_COMB, s, [&] {
                    return launch_blk_comb_dual(pool, l_as, m, k, dY, pool, l_axn, l_apn, k, n, s);
                }, true, bytes);
            if (e != hipSuccess) return hip_fail("ritz vectors");
        } else {
            if ((e = comb(pool, l_s, m, dY, pool, l_xn, k, nullptr)) != hipSuccess) return hip_fail("ritz vectors");
            if ((e = comb(pool, l_as, m, dY, pool, l_axn, k, nullptr)) != hipSuccess) return hip_fail("ritz vectors");
            const double* dYk = dY + static_cast<size_t>(k) * k;
            if ((e = comb(pool, l_sk, m - k, dYk, pool, l_pn, k, nullptr)) != hipSuccess) return hip_fail("directions");
            if ((e = comb(pool, l_ask, m - k, dYk, pool, l_apn, k, nullptr)) != hipSuccess)
                return hip_fail("directions");
        }
        par = nx;
        has_p = true;
    }
    // unit Ritz vectors signed by <u_r, X0[r]>, written to d_evecs
    {
        lists.room(kPhaseLists);
        const int32_t* l_x = lists.get(c_x[par]);
        const int32_t* l_x0 = lists.get(c_x0);
        if ((e = lists.flush(s)) != hipSuccess) return hip_fail("output");
        if ((e = gram(pool, l_x, k, pool, l_x, k, true, dH)) != hipSuccess) return hip_fail("output");
        if ((e = gram(pool, l_x, k, d_X0, l_x0, k, false, dH + static_cast<size_t>(k) * k)) != hipSuccess)
            return hip_fail("output");
        HIP_TRY(hipStreamSynchronize(s));
        std::vector<double> Yo(static_cast<size_t>(k) * k, 0.0);
        for (int r = 0; r < k; ++r) {
            const double nu = std::sqrt(hH[r * k + r]);
            const double sgn = hH[static_cast<size_t>(k) * k + r * k + r] < 0.0 ? -1.0 : 1.0;
            Yo[r * k + r] = 1.0 / (sgn * nu);
        }
        ar.reset();
        const double* dYo = ar.put(Yo.data(), Yo.size(), e);
        if (e != hipSuccess) return hip_fail("output");
        const double* dth = ar.put(theta.data(), theta.size(), e);
        if (e != hipSuccess) return hip_fail("output");
        HIP_TRY(ar.flush(s));
        if ((e = comb(pool, l_x, k, dYo, d_evecs, l_x0, k, nullptr)) != hipSuccess) return hip_fail("output");
        HIP_TRY(hipMemcpyAsync(d_evals, dth, sizeof(double) * k, hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipStreamSynchronize(s));
        ar.reset();
    }
    info->iterations = it;
    info->state = state;
    info->restarts = 0;
    double mr = 0.0;
    for (int r = 0; r < k; ++r) mr = std::max(mr, res[r]);
    info->max_res = mr;
    hipError_t te = timing_collect();
    if (te != hipSuccess) return fail(SLA_ERR_HIP, "timing collect: %s", hipGetErrorString(te));
    return SLA_OK;
}

sla_status sla_eigsh_backward(const sla_csr* Ac, int32_t k, const double* d_evecs, const double* d_gevals,
                              double* d_gvals, void* stream)
{
    sla_status st = check_common(Ac, 1);
    if (st != SLA_OK) return st;
    if (k < 1 || k > SLA_EIG_MAX_K) return fail(SLA_ERR_INVALID_ARG, "k must be in [1, %d]", SLA_EIG_MAX_K);
    if (!d_evecs || !d_gevals || (!d_gvals && Ac->nnz > 0)) return fail(SLA_ERR_INVALID_ARG, "NULL argument");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed(SLA_K_LZ_RITZ, s, [&] {
        return launch_eig_grad(Ac->krp, Ac->krp_bits, Ac->col, d_evecs, d_gevals, k, Ac->n_rows, Ac->nnz, d_gvals,
                               s);
    });
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "eigsh backward launch: %s", hipGetErrorString(e));
    return SLA_OK;
}

sla_status sla_list_destroy(sla_list* L)
{
    if (!L) return SLA_OK;
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != L->device) (void)hipSetDevice(L->device);
    (void)hipDeviceSynchronize();
    if (L->packed) (void)sla_csr_destroy(L->packed);
    if (L->rp) (void)dev_free(L->rp);
    if (L->col) (void)dev_free(L->col);
    if (L->d_wg) (void)dev_free(L->d_wg);
    if (L->d_tiles) (void)dev_free(L->d_tiles);
    if (L->d_rend) (void)dev_free(L->d_rend);
    if (L->stage) (void)dev_free(L->stage);
    if (prev >= 0 && prev != L->device) (void)hipSetDevice(prev);
    delete L;
    return SLA_OK;
}

sla_status sla_list_create(sla_list** out, int32_t items, const int64_t* n, const int64_t* nnz,
                           const void* const* d_row_ptr, int32_t row_ptr_bits, const int32_t* const* d_col,
                           uint32_t flags, void* stream)
{
    if (!out) return fail(SLA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (items < 1 || items > (1 << 20)) return fail(SLA_ERR_INVALID_ARG, "items must be in [1, 2^20] (got %d)", items);
    if (!n || !nnz || !d_row_ptr || !d_col) return fail(SLA_ERR_INVALID_ARG, "NULL array");
    if (row_ptr_bits != 32 && row_ptr_bits != 64) return fail(SLA_ERR_INVALID_ARG, "row_ptr_bits must be 32 or 64");
    if (flags & ~(SLA_SYMMETRIC | SLA_EAGER_TRANSPOSE)) return fail(SLA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // everything allocated below is released by sla_list_destroy if creation fails
    struct Guard {
        sla_list* p;
        ~Guard() { if (p) (void)sla_list_destroy(p); }
    } guard{new (std::nothrow) sla_list};
    sla_list* const L = guard.p;
    if (!L) return fail(SLA_ERR_OOM, "host allocation failed");
    HIP_TRY(hipGetDevice(&L->device));
    L->items = items;
    L->flags = flags;
    int64_t tiles = 0, ents = 0;
    std::vector<int64_t> tile0(items + 1), rend(items);
    for (int32_t i = 0; i < items; ++i) {
        if (n[i] < 1 || nnz[i] < 0 || !d_row_ptr[i] || (nnz[i] > 0 && !d_col[i]))
            return fail(SLA_ERR_INVALID_ARG, "item %d: n must be >= 1, nnz >= 0, arrays non-NULL", i);
        if (row_ptr_bits == 32 && nnz[i] >= (int64_t(1) << 31))
            return fail(SLA_ERR_INVALID_ARG, "item %d: nnz does not fit 32-bit row pointers", i);
        L->n.push_back(n[i]);
        L->nnz.push_back(nnz[i]);
        L->r0.push_back(tiles * kTile);
        L->e0.push_back(ents);
        tile0[i] = tiles;
        rend[i] = tiles * kTile + n[i];
        tiles += (n[i] + kTile - 1) / kTile;
        ents += nnz[i];
    }
    tile0[items] = tiles;
    L->n_total = tiles * kTile;
    L->nnz_total = ents;
    if (L->n_total >= (int64_t(1) << 31)) return fail(SLA_ERR_UNSUPPORTED, "packed rows exceed 2^31");
    // each item's own pattern is checked first: a column of one item must not reach
    // into another item's rows
    int32_t* d_chk = nullptr;
    sla_status st = dev_alloc(reinterpret_cast<void**>(&d_chk), sizeof(int32_t) * kChkCount * items);
    if (st != SLA_OK) return st;
    std::vector<int32_t> h_chk(static_cast<size_t>(kChkCount) * items);
    for (int32_t i = 0; i < items; ++i) {
        int32_t* c = &h_chk[static_cast<size_t>(kChkCount) * i];
        c[kChkErr] = 0, c[kChkTileMax] = 0, c[kChkRowMax] = 0, c[kChkFarMin] = INT32_MAX, c[kChkFarMax] = 0;
    }
    hipError_t e = hipMemcpyAsync(d_chk, h_chk.data(), sizeof(int32_t) * h_chk.size(), hipMemcpyHostToDevice, s);
    for (int32_t i = 0; i < items && e == hipSuccess; ++i)
        e = launch_validate(d_row_ptr[i], row_ptr_bits, d_col[i], n[i], n[i], nnz[i], d_chk + kChkCount * i, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(h_chk.data(), d_chk, sizeof(int32_t) * h_chk.size(), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    (void)dev_free(d_chk);
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "list validation: %s", hipGetErrorString(e));
    for (int32_t i = 0; i < items; ++i)
        if (h_chk[static_cast<size_t>(kChkCount) * i + kChkErr] != 0)
            return fail(SLA_ERR_INVALID_CSR, "item %d: malformed CSR pattern (code %d)", i,
                        h_chk[static_cast<size_t>(kChkCount) * i + kChkErr]);
    // packed pattern
    const int out_bits = ents < (int64_t(1) << 31) ? 32 : 64;
    if ((st = dev_alloc(&L->rp, static_cast<size_t>(L->n_total + 1) * (out_bits / 8))) != SLA_OK) return st;
    if ((st = dev_alloc(reinterpret_cast<void**>(&L->col), std::max<size_t>(4, 4 * static_cast<size_t>(ents)))) !=
        SLA_OK)
        return st;
    for (int32_t i = 0; i < items; ++i) {
        const int64_t rows_padded = (tile0[i + 1] - tile0[i]) * kTile;
        e = launch_pack_pattern(d_row_ptr[i], row_ptr_bits, d_col[i], n[i], nnz[i], L->r0[i], L->e0[i], rows_padded,
                                L->rp, out_bits, L->col, s);
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "list packing: %s", hipGetErrorString(e));
    }
    if ((st = sla_csr_create(&L->packed, L->n_total, L->n_total, ents, L->rp, out_bits, L->col, flags, stream)) !=
        SLA_OK)
        return st;
    L->packed->band = 0;          // the list solve runs the plain or split SpMV
    L->packed->group_ok = false;
    // Workgroups per item.  Every launch of the solve lasts as long as its busiest
    // workgroup, so the split minimises the most tiles any workgroup walks, m, over
    // grids that fit the GPU once (n_cu x the SpMV's occupancy): each item gets the
    // fewest workgroups with at most m tiles each, a multiple of 8 from 8 up where the
    // item has the tiles (its workgroups on one XCD then sweep a contiguous eighth of
    // its tiles, block_coord; an eighth holds at most ceil(ti / 8) tiles).
    const int per_cu = cg_blocks_per_cu(L->packed->krp_bits, L->packed->cap, L->n_total, L->packed->split);
    const int64_t capacity = std::max<int64_t>(items, static_cast<int64_t>(L->packed->n_cu) * per_cu);
    auto count_for = [](int64_t ti, int64_t m) {
        int64_t gi = std::max<int64_t>(1, (ti + m - 1) / m);
        if (gi >= 8) {
            int64_t g8 = (gi + 7) & ~int64_t(7);
            while (g8 <= ti && ((ti + 7) / 8 + g8 / 8 - 1) / (g8 / 8) > m) g8 += 8;
            if (g8 <= ti) gi = g8;
        }
        return std::min<int64_t>(gi, ti);
    };
    auto total_for = [&](int64_t m) {
        int64_t acc = 0;
        for (int32_t i = 0; i < items; ++i) acc += count_for(tile0[i + 1] - tile0[i], m);
        return acc;
    };
    int64_t mlo = 1, mhi = 1;
    for (int32_t i = 0; i < items; ++i) mhi = std::max<int64_t>(mhi, tile0[i + 1] - tile0[i]);
    while (mlo < mhi) {   // smallest m whose grid fits (m = the largest item's tiles: one each)
        const int64_t mid = (mlo + mhi) / 2;
        if (total_for(mid) <= capacity) mhi = mid;
        else mlo = mid + 1;
    }
    std::vector<int32_t> wg(items + 1);
    int64_t acc = 0;
    for (int32_t i = 0; i < items; ++i) {
        wg[i] = static_cast<int32_t>(acc);
        acc += count_for(tile0[i + 1] - tile0[i], mlo);
    }
    if (acc >= (int64_t(1) << 31)) return fail(SLA_ERR_UNSUPPORTED, "too many workgroups");
    wg[items] = static_cast<int32_t>(acc);
    L->total_wg = static_cast<int32_t>(acc);
    if ((st = dev_alloc(reinterpret_cast<void**>(&L->d_wg), sizeof(int32_t) * (items + 1))) != SLA_OK) return st;
    if ((st = dev_alloc(reinterpret_cast<void**>(&L->d_tiles), sizeof(int64_t) * (items + 1))) != SLA_OK) return st;
    if ((st = dev_alloc(reinterpret_cast<void**>(&L->d_rend), sizeof(int64_t) * items)) != SLA_OK) return st;
    HIP_TRY(hipMemcpyAsync(L->d_wg, wg.data(), sizeof(int32_t) * (items + 1), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(L->d_tiles, tile0.data(), sizeof(int64_t) * (items + 1), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(L->d_rend, rend.data(), sizeof(int64_t) * items, hipMemcpyHostToDevice, s));
    HIP_TRY(hipStreamSynchronize(s));
    *out = L;
    guard.p = nullptr;
    return SLA_OK;
}

sla_status sla_list_col_bits(const sla_list* L, int32_t* col_bits)
{
    if (!L) return fail(SLA_ERR_INVALID_ARG, "list is NULL");
    return sla_csr_col_bits(L->packed, col_bits);
}

sla_status sla_list_info(const sla_list* L, int64_t* n_total, int64_t* nnz_total, int32_t* workgroups)
{
    if (!L) return fail(SLA_ERR_INVALID_ARG, "list is NULL");
    if (n_total) *n_total = L->n_total;
    if (nnz_total) *nnz_total = L->nnz_total;
    if (workgroups) *workgroups = L->total_wg;
    return SLA_OK;
}

namespace {

// Staging of a list solve: packed values, three packed vectors, packed gradient.
sla_status list_stage(sla_list* L, bool want_grad, double** vals, double** v0, double** v1, double** v2,
                      double** gv)
{
    const size_t sv = align256(sizeof(double) * std::max<int64_t>(L->nnz_total, 1));
    const size_t sn = align256(sizeof(double) * L->n_total);
    const size_t need = 2 * sv + 3 * sn;
    if (need > L->stage_bytes) {
        if (L->stage) {
            HIP_TRY(hipDeviceSynchronize());
            HIP_TRY(dev_free(L->stage));
            L->stage = nullptr;
            L->stage_bytes = 0;
        }
        sla_status st = dev_alloc(reinterpret_cast<void**>(&L->stage), need);
        if (st != SLA_OK) return st;
        L->stage_bytes = need;
    }
    char* p = reinterpret_cast<char*>(L->stage);
    *vals = reinterpret_cast<double*>(p);
    *v0 = reinterpret_cast<double*>(p + sv);
    *v1 = reinterpret_cast<double*>(p + sv + sn);
    *v2 = reinterpret_cast<double*>(p + sv + 2 * sn);
    *gv = want_grad ? reinterpret_cast<double*>(p + sv + 3 * sn) : nullptr;
    return SLA_OK;
}

// Copy each item's values / vector into the packed layout (vectors zero-padded).
sla_status list_pack(const sla_list* L, const double* const* items, double* out, bool values, hipStream_t s)
{
    if (!values) HIP_TRY(hipMemsetAsync(out, 0, sizeof(double) * L->n_total, s));
    for (int32_t i = 0; i < L->items; ++i) {
        const int64_t cnt = values ? L->nnz[i] : L->n[i];
        if (cnt == 0) continue;
        if (!items[i]) return fail(SLA_ERR_INVALID_ARG, "item %d: NULL array", i);
        HIP_TRY(hipMemcpyAsync(out + (values ? L->e0[i] : L->r0[i]), items[i], sizeof(double) * cnt,
                               hipMemcpyDeviceToDevice, s));
    }
    return SLA_OK;
}

sla_status list_unpack(const sla_list* L, const double* in, double* const* items, bool values, hipStream_t s)
{
    for (int32_t i = 0; i < L->items; ++i) {
        const int64_t cnt = values ? L->nnz[i] : L->n[i];
        if (cnt == 0) continue;
        if (!items[i]) return fail(SLA_ERR_INVALID_ARG, "item %d: NULL output", i);
        HIP_TRY(hipMemcpyAsync(items[i], in + (values ? L->e0[i] : L->r0[i]), sizeof(double) * cnt,
                               hipMemcpyDeviceToDevice, s));
    }
    return SLA_OK;
}

ListPlan plan_of(const sla_list* L)
{
    return ListPlan{L->d_wg, L->d_tiles, L->d_rend, L->items, L->total_wg};
}

sla_status check_list(const sla_list* L, const sla_cg_opts* opts)
{
    if (!L) return fail(SLA_ERR_INVALID_ARG, "list is NULL");
    sla_status st = check_opts(opts);
    if (st != SLA_OK) return st;
    if (opts->flags & SLA_BICGSTAB) return fail(SLA_ERR_UNSUPPORTED, "list solves take CG or Jacobi CG only");
    return check_device(L->packed);
}

}  // namespace

sla_status sla_list_solve(const sla_list* Lc, const double* const* d_vals, const double* const* d_b,
                          double* const* d_x, const sla_cg_opts* opts, sla_cg_info* d_info, void* stream)
{
    sla_status st = check_list(Lc, opts);
    if (st != SLA_OK) return st;
    if (!d_vals || !d_b || !d_x || !d_info) return fail(SLA_ERR_INVALID_ARG, "NULL array");
    sla_list* L = const_cast<sla_list*>(Lc);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lk(L->mu);
    std::lock_guard<std::mutex> lk2(L->packed->mu);
    double *vals, *b, *x, *unused, *gv;
    if ((st = list_stage(L, false, &vals, &b, &x, &unused, &gv)) != SLA_OK) return st;
    if ((st = list_pack(L, d_vals, vals, true, s)) != SLA_OK) return st;
    if ((st = list_pack(L, d_b, b, false, s)) != SLA_OK) return st;
    sla_csr* A = L->packed;
    const ListPlan plan = plan_of(L);
    st = run_cg(A, A->krp, A->col, A->cap, 0, 0, A->split, 1, vals, b, x, opts, d_info, s, &plan);
    if (st != SLA_OK) return st;
    if ((st = list_unpack(L, x, d_x, false, s)) != SLA_OK) return st;
    if (!(opts->flags & SLA_FIXED_ITERS)) {
        hipError_t e = timing_collect();
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "timing collect: %s", hipGetErrorString(e));
    }
    return SLA_OK;
}

sla_status sla_list_solve_backward(const sla_list* Lc, const double* const* d_vals, const double* const* d_x,
                                   const double* const* d_gx, double* const* d_gb, double* const* d_gvals,
                                   const sla_cg_opts* opts, sla_cg_info* d_info, void* stream)
{
    sla_status st = check_list(Lc, opts);
    if (st != SLA_OK) return st;
    if (!d_vals || !d_gx || !d_gb || !d_info || (d_gvals && !d_x)) return fail(SLA_ERR_INVALID_ARG, "NULL array");
    sla_list* L = const_cast<sla_list*>(Lc);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lk(L->mu);
    std::lock_guard<std::mutex> lk2(L->packed->mu);
    double *vals, *g, *lam, *xp, *gv;
    if ((st = list_stage(L, d_gvals != nullptr, &vals, &g, &lam, &xp, &gv)) != SLA_OK) return st;
    if ((st = list_pack(L, d_vals, vals, true, s)) != SLA_OK) return st;
    if ((st = list_pack(L, d_gx, g, false, s)) != SLA_OK) return st;
    sla_csr* A = L->packed;
    const ListPlan plan = plan_of(L);
    if (A->flags & SLA_SYMMETRIC) {
        st = run_cg(A, A->krp, A->col, A->cap, 0, 0, A->split, 1, vals, g, lam, opts, d_info, s, &plan);
    } else {
        // the transpose of the block-diagonal packed pattern is block-diagonal on the
        // same row blocks, so the same plan applies
        if ((st = ensure_transpose(A, s)) != SLA_OK) return st;
        const double* vt = nullptr;
        if ((st = ensure_vals_t(A, 1, vals, s, &vt)) != SLA_OK) return st;
        st = run_cg(A, A->row_ptr_t, A->col_t, A->cap_t, 0, 0, A->split, 1, vt, g, lam, opts, d_info, s, &plan);
    }
    if (st != SLA_OK) return st;
    if ((st = list_unpack(L, lam, d_gb, false, s)) != SLA_OK) return st;
    if (d_gvals) {
        if ((st = list_pack(L, d_x, xp, false, s)) != SLA_OK) return st;
        hipError_t e = timed(SLA_K_PATTERN_OUTER, s, [&] {
            return launch_pattern_outer(A->krp, A->krp_bits, A->col, -1.0, lam, A->n_rows, xp, A->n_cols, gv,
                                        A->n_rows, A->nnz, 1, s);
        });
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "gradient scatter launch: %s", hipGetErrorString(e));
        if ((st = list_unpack(L, gv, d_gvals, true, s)) != SLA_OK) return st;
    }
    if (!(opts->flags & SLA_FIXED_ITERS)) {
        hipError_t e = timing_collect();
        if (e != hipSuccess) return fail(SLA_ERR_HIP, "timing collect: %s", hipGetErrorString(e));
    }
    return SLA_OK;
}

sla_status sla_timing_enable(int32_t enable)
{
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing = enable != 0;
    return SLA_OK;
}

sla_status sla_set_allocator(sla_alloc_fn alloc, sla_free_fn free_fn, void* ctx)
{
    if ((alloc == nullptr) != (free_fn == nullptr))
        return fail(SLA_ERR_INVALID_ARG, "give both alloc and free, or neither");
    std::lock_guard<std::mutex> lk(g_amu);
    g_hook = AllocHook{alloc, free_fn, ctx};
    return SLA_OK;
}

sla_status sla_timing_reset(void)
{
    std::lock_guard<std::mutex> lk(g_tmu);
    for (int i = 0; i < SLA_K_COUNT; ++i) {
        g_launches[i] = 0;
        g_ms[i] = 0.0;
        g_bytes[i] = 0.0;
    }
    return SLA_OK;
}

sla_status sla_timing_collect(void)
{
    hipError_t e = timing_collect();
    if (e != hipSuccess) return fail(SLA_ERR_HIP, "timing collect: %s", hipGetErrorString(e));
    return SLA_OK;
}

sla_status sla_timing_query(int32_t kernel, int64_t* launches, double* total_ms)
{
    if (kernel < 0 || kernel >= SLA_K_COUNT) return fail(SLA_ERR_INVALID_ARG, "unknown kernel id %d", kernel);
    std::lock_guard<std::mutex> lk(g_tmu);
    if (launches) *launches = g_launches[kernel];
    if (total_ms) *total_ms = g_ms[kernel];
    return SLA_OK;
}

sla_status sla_timing_query_bytes(int32_t kernel, double* bytes)
{
    if (kernel < 0 || kernel >= SLA_K_COUNT) return fail(SLA_ERR_INVALID_ARG, "unknown kernel id %d", kernel);
    if (!bytes) return fail(SLA_ERR_INVALID_ARG, "NULL argument");
    std::lock_guard<std::mutex> lk(g_tmu);
    *bytes = g_bytes[kernel];
    return SLA_OK;
}

}  // extern "C"
