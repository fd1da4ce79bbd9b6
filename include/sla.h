/*
 * sla.h -- C ABI of the MI355X (gfx950) sparse CG solve and its adjoint.
 *
 * The operations follow torch-sla: Differentiable Sparse Linear Algebra with
 * Adjoint Solvers and Sparse Tensor Parallelism for PyTorch:
 *   - the API calls .matvec and .solve(b), with gradients flowing to the matrix
 *     values and to b (paperpeel page, section 3.1 "API" and "Bridging backends
 *     into autograd"; gist.science summaries, Methodology item 1);
 *   - an explicit val/row/col operator (paperpeel, section "Operator
 *     representation: explicit vs. implicit"), stored here as CSR;
 *   - a SparseTensor is one matrix or a batch sharing one pattern (gist.science
 *     summaries, Methodology item 1; paperpeel section 3.1 "Typed sparse-tensor
 *     hierarchy"): every call below takes `batch` systems whose values are
 *     [batch][nnz] over one pattern -- the batched shared-pattern variants;
 *   - the solve is the pytorch-native backend's conjugate gradient, here
 *     without preconditioner (paperpeel sections 1 and 3.1; section 3.3
 *     "Distributed Krylov solvers" for one SpMV and the inner products <r,r>,
 *     <p,Ap> per iteration);
 *   - the backward pass solves A^T lambda = dL/dx and returns dL/db = lambda and
 *     dL/dA_ij = -lambda_i x_j on the stored entries only (gist.science Hindi and
 *     Japanese summaries, Methodology item 2, linear-systems bullet; paperpeel
 *     section 3.2.3 "Complexity": one adjoint solve of the same size and pattern
 *     plus an O(nnz) outer product).
 *
 * Conventions for every call:
 *   - Pointers named d_* or documented "device" are device pointers on the
 *     current HIP device; everything else is host memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued on it.  sla_solve / sla_solve_backward with a residual
 *     test block the calling host thread until the iterations have finished on
 *     the stream (they poll a device counter once per chunk of iterations);
 *     everything else returns after enqueueing.
 *   - The caller owns every array it passes.  A handle borrows row_ptr and
 *     col_idx: they must stay valid and unchanged until sla_csr_destroy.  The
 *     library owns the handle's analysis data, an optional transposed pattern,
 *     and a per-handle workspace (CG vectors and reduction partials, O(n + nnz)
 *     per system, independent of the iteration count) which it allocates on
 *     first use and frees in sla_csr_destroy.
 *   - Calls that share one handle must not overlap in time (use one stream per
 *     handle, or serialise): they share its workspace.
 *   - Errors: argument problems are returned as sla_status before anything is
 *     enqueued.  Numerical outcomes of a solve (converged, budget reached,
 *     breakdown) are per-system states written into the device info array,
 *     never return codes.  sla_last_error() gives a message for the calling
 *     thread's most recent non-OK status.
 */
#ifndef SLA_H
#define SLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SLA_OK = 0,
    SLA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad flag, batch < 1, ... */
    SLA_ERR_INVALID_CSR = 2,   /* row_ptr not monotone / not starting at 0 / not ending at nnz,
                                  a column out of range, or columns not strictly ascending */
    SLA_ERR_UNSUPPORTED = 3,   /* e.g. a solve on a non-square matrix */
    SLA_ERR_OOM = 4,           /* device allocation of library-owned memory failed */
    SLA_ERR_HIP = 5            /* a HIP runtime call failed; see sla_last_error() */
} sla_status;

/* Per-system outcome of a solve, in sla_cg_info.state (same numbers as the oracle). */
enum {
    SLA_CONVERGED = 0,   /* |r_k| <= max(rtol |rhs|, atol) with r_k the recurrence residual */
    SLA_MAX_ITER = 1,    /* iteration budget reached (always the outcome with SLA_FIXED_ITERS) */
    SLA_NOT_SPD = 2,     /* p^T A p <= 0 (or, with SLA_JACOBI, a diagonal entry <= 0 or missing) */
    SLA_NAN = 3,         /* p^T A p is NaN (or, with SLA_JACOBI, a NaN diagonal entry;
                            with SLA_BICGSTAB, <rh, A p>, <t, s> or <t, t> is NaN) */
    SLA_BREAKDOWN = 4    /* SLA_BICGSTAB only: <rh, A p> = 0, <t, t> = 0, or a zero
                            <rh, r> or omega at the start of an iteration */
};

/* sla_csr_create flags */
#define SLA_SYMMETRIC        1u  /* caller asserts A == A^T exactly: the adjoint reuses A */
#define SLA_EAGER_TRANSPOSE  2u  /* build the transposed pattern now instead of on first need */

/* sla_cg_opts.flags */
#define SLA_FIXED_ITERS      1u  /* skip the residual test: run exactly max_iter iterations */
/*
 * Jacobi-preconditioned CG, M = diag(A) (paperpeel page, section 4.1, Table 3: the
 * pages' CG runs with a Jacobi preconditioner).  Per iteration z = M^{-1} r (a
 * division by the stored diagonal entry), rho = <r, z>, p = z + beta p; the stop test
 * stays |r| <= max(rtol |rhs|, atol) on the recurrence residual, and
 * residual_history still records |r_k|.  A missing or non-positive diagonal entry
 * stops the system with SLA_NOT_SPD before the first iteration, a NaN one with
 * SLA_NAN (a zero right-hand side stops first, converged).  The adjoint solve uses
 * the same preconditioner (A^T has the same diagonal).
 */
#define SLA_JACOBI           2u
/*
 * BiCGStab instead of CG, for nonsymmetric (and SPD) systems: van der Vorst's method
 * (Bi-CGSTAB, SIAM J. Sci. Stat. Comput. 13(2), 1992), the second iterative method of
 * the pages' backends (paperpeel page, section 1; section 3.1 "Five backends and
 * auto-dispatch").  x0 = 0, shadow residual rh = b, no preconditioner (not combinable
 * with SLA_JACOBI: SLA_ERR_INVALID_ARG).  Iteration k:
 *   stop if |r| <= max(rtol |rhs|, atol) or k = max_iter;
 *   k > 0: beta = (rho_k / rho_{k-1}) (alpha / omega), p = r + beta (p - omega v),
 *          with rho_k = <rh, r>;
 *   v = A p, alpha = rho_k / <rh, v>, s = r - alpha v, t = A s,
 *   |s| <= threshold: x += alpha p, stop (converged; counts as iteration k + 1);
 *   omega = <t, s> / <t, t>, x += alpha p + omega s, r = s - omega t.
 * iterations counts the products A p; residual_history records |r_k| (|s| for a stop
 * half-way).  Breakdowns stop with SLA_BREAKDOWN (or SLA_NAN) and the x before the
 * failing iteration.  The adjoint solve of sla_solve_backward uses BiCGStab on A^T
 * (on A for an SLA_SYMMETRIC handle).
 */
#define SLA_BICGSTAB         4u

typedef struct sla_csr sla_csr;   /* opaque handle: one sparsity pattern */

/*
 * Device memory of the library (handle workspaces, transposes, Lanczos and LOBPCG
 * vectors, list staging) from a caller's allocator, e.g. a framework's caching
 * allocator, instead of hipMalloc/hipFree.  Not a passage of the pages: the interface
 * by which a host framework keeps the library's memory inside its own pool.
 *   alloc(bytes, stream, ctx) returns device memory of at least `bytes` on the current
 *     device, or NULL (the calling entry point then fails with SLA_ERR_OOM); stream is
 *     passed as NULL: the library reuses its workspaces across calls and streams.
 *   free(ptr, stream, ctx) takes back a block of alloc; the library synchronizes the
 *     device first, so the block is idle on every stream.
 * Both NULL restores hipMalloc/hipFree; one NULL is SLA_ERR_INVALID_ARG.  Applies to
 * allocations made after the call; every block is freed through the allocator that
 * made it.  Process-wide; the callbacks must be thread-safe if the library is used
 * from several threads.
 */
typedef void* (*sla_alloc_fn)(size_t bytes, void* stream, void* ctx);
typedef void (*sla_free_fn)(void* ptr, void* stream, void* ctx);
sla_status sla_set_allocator(sla_alloc_fn alloc, sla_free_fn free, void* ctx);

typedef struct {
    double rtol;                 /* relative tolerance on |r| / |rhs| (>= 0) */
    double atol;                 /* absolute tolerance on |r| (>= 0) */
    int64_t max_iter;            /* iteration budget (>= 0) */
    int32_t check_every;         /* iterations between host polls of the stop counter (0 = default 32) */
    uint32_t flags;              /* SLA_FIXED_ITERS | SLA_JACOBI | SLA_BICGSTAB */
    double* residual_history;    /* device, nullable: [batch][max_iter + 1], entry k = |r_k| */
} sla_cg_opts;

typedef struct {
    int64_t iterations;          /* number of products A p performed */
    double res_norm;             /* |r| of the recurrence residual at exit */
    double rhs_norm;             /* |b| (forward) or |dL/dx| (backward) */
    int32_t state;               /* SLA_CONVERGED, SLA_MAX_ITER, SLA_NOT_SPD, SLA_NAN or SLA_BREAKDOWN */
    int32_t reserved;
} sla_cg_info;                   /* 32 bytes; device arrays of these have one entry per system */

/*
 * Create a handle for an n_rows x n_cols CSR pattern (paperpeel section
 * "Operator representation": explicit val/row/col storage).
 *   d_row_ptr  device, n_rows + 1 entries of int32 (row_ptr_bits = 32) or int64 (64);
 *              d_row_ptr[0] = 0, non-decreasing, d_row_ptr[n_rows] = nnz.
 *   d_col_idx  device int32 [nnz], strictly ascending within each row, in [0, n_cols).
 * The pattern is validated on the device (one pass and one host synchronisation
 * on `stream`); a malformed pattern returns SLA_ERR_INVALID_CSR and no handle.
 * The analysis (per-tile entry counts that pick the SpMV variant, and the band test
 * below) is computed here.
 * n_rows, n_cols < 2^31; nnz < 2^31 with 32-bit row pointers.  nnz may be 0.
 *
 * Band test: a square pattern with n_rows < 2^29 and nnz < 2^31 is banded with line
 * stride S when every stored entry (i, c) has |c - i| <= 8 or S - 8 <= |c - i| <= S, where S is the
 * largest |c - i| (5- and 9-point stencils of a grid in natural order, S = line length
 * or line length + 1), S >= 272, rows hold at most 16 entries, and S is at least the
 * minimum stride: 2048 by default, or the value of the environment variable
 * SLA_BAND_MIN_STRIDE (read at each create).  The CG SpMV of a banded pattern walks
 * the rows line by line and reads the operand from LDS; results are the same to the
 * last bit per row as the plain SpMV's.
 *
 * Column offsets: a square pattern with n_rows < 2^29, 32-bit row pointers (or nnz <
 * 2^31, when the library keeps a 32-bit copy) and every |c - i| <= 32512 also gets
 * 16-bit column offsets (c minus the first row of the entry's 256-row tile, 2 nnz
 * bytes of device memory), which the plain CG and BiCGStab SpMV read in place of
 * d_col_idx: 2 bytes less per stored entry in every product, the same sums to the
 * last bit.  A banded pattern also gets offsets from the first row of each row's
 * window of the line-walking SpMV (another 2 nnz bytes).  The environment variable SLA_COL16=0 (read at each create) turns them
 * off.  When the library builds such a copy (offsets, 32-bit row pointers) the call
 * synchronises `stream` once more before it returns.  The pattern arrays must stay
 * unchanged while the handle lives.
 */
sla_status sla_csr_create(sla_csr** out, int64_t n_rows, int64_t n_cols, int64_t nnz,
                          const void* d_row_ptr, int32_t row_ptr_bits, const int32_t* d_col_idx,
                          uint32_t flags, void* stream);

/* Destroy a handle and free everything the library allocated for it (synchronises the device). */
sla_status sla_csr_destroy(sla_csr* A);

/* Width in bits of the column indices the plain and banded CG / BiCGStab SpMV read: 16
 * when the handle holds 16-bit column offsets (see sla_csr_create), else 32. */
sla_status sla_csr_col_bits(const sla_csr* A, int32_t* col_bits);
/* Diagonals of the banded CG SpMV's diagonal layout (set at sla_csr_create): for a
 * banded pattern (sla_csr_analysis band_stride > 0) whose stored offsets c - i take at
 * most 16 distinct values, that number (5 for a 5-point grid stencil), and the CG
 * solves on the handle's own pattern read the values in that layout: one value per
 * diagonal and row, copied from the CSR values once per solve, and a per-row mask of the
 * diagonals the row stores.  0: the staged CSR banded SpMV (more diagonals, not banded,
 * or SLA_DIA=0 in the environment at create).  Row sums are the same either way. */
sla_status sla_csr_diagonals(const sla_csr* A, int32_t* n_diagonals);
/* Operand window of the grouped batch SpMV (batches of at least 8 systems, a multiple
 * of 4, on split-schedule patterns; paperpeel section 3.1: batched SparseTensor).  Those
 * solves run on a reverse Cuthill-McKee order of the pattern, computed at the handle's
 * first grouped solve.  When every entry of that order lies within 448 rows of its
 * row, each workgroup of the SpMV keeps the operand rows around its tile in LDS and
 * reads the gathers there; *halo_rows is then that halo (rows on each side, a multiple
 * of 64).  0: the SpMV gathers from memory (bandwidth above 448, the reordering off, or
 * SLA_GCG_WINDOW=0 in the environment at create), or no grouped solve has run yet.
 * Row sums are the same either way. */
sla_status sla_csr_group_window(const sla_csr* A, int32_t* halo_rows);

/* Shape and workspace queries (host outputs; any pointer may be NULL). */
sla_status sla_csr_info(const sla_csr* A, int64_t* n_rows, int64_t* n_cols, int64_t* nnz,
                        int32_t* row_ptr_bits, uint32_t* flags, int64_t* workspace_bytes);

/*
 * Results of the pattern analysis done at create (host outputs; any pointer may be
 * NULL): the most entries of any row and of any 256-row tile, the LDS capacity (in
 * entries) of the SpMV variant the CG solve uses, the line stride S of a banded
 * pattern (0 if the pattern is not banded, see sla_csr_create), and whether the CG
 * solve uses the split schedule (1) or the fused one (0).
 *
 * Schedules.  Fused: one SpMV kernel forms p_k = r_k + beta p_{k-1} at every gathered
 * column, applies the deferred x update and computes q = A p_k and p_k^T q; then one
 * update kernel.  Split: a streaming kernel first forms p_k and the x update, so the
 * SpMV gathers p_k alone (half the gather requests, one more vector pass).  A pattern
 * that is not banded but has an entry at |c - i| >= 4096 takes the split schedule
 * (unstructured gathers); the environment variable SLA_CG_SCHEDULE ("fused" or
 * "split", read at each create) overrides the choice.  Banded patterns use their own
 * SpMV.  The schedules give the same row sums to the last bit.
 */
sla_status sla_csr_analysis(const sla_csr* A, int32_t* row_max, int32_t* tile_max, int32_t* spmv_cap,
                            int64_t* band_stride, int32_t* cg_split);

/*
 * y = A x for `batch` systems sharing the pattern (paperpeel section 3.3: the
 * SpMV; section 3.1: .matvec).
 *   d_vals [batch][nnz], d_x [batch][n_cols], d_y [batch][n_rows] (device, fp64).
 * Row i is summed over its stored entries in ascending position order.
 */
sla_status sla_matvec(const sla_csr* A, int64_t batch, const double* d_vals, const double* d_x,
                      double* d_y, void* stream);

/*
 * Backward of y = A x: d_gx = A^T gy (nullable) and d_gvals[k] = gy[row(k)] * x[col(k)]
 * (nullable), per system.  A^T is A when the handle is SLA_SYMMETRIC, otherwise the
 * transposed pattern (built on first need).
 *   d_gy [batch][n_rows], d_gx [batch][n_cols], d_gvals [batch][nnz].
 */
sla_status sla_matvec_backward(const sla_csr* A, int64_t batch, const double* d_vals,
                               const double* d_x, const double* d_gy, double* d_gx,
                               double* d_gvals, void* stream);

/*
 * Solve A x = b by unpreconditioned conjugate gradients from x0 = 0, for `batch`
 * independent systems sharing the pattern (paperpeel sections 1, 3.1, 3.3).
 *   d_vals [batch][nnz], d_b [batch][n], d_x [batch][n] (output), d_info [batch] (output).
 * Each iteration: q = A p, sigma = p^T q, alpha = rho / sigma, x += alpha p,
 * r -= alpha q, rho' = r^T r, stop test, beta = rho' / rho, p = r + beta p.
 * Each system stops on its own test (|r| <= max(rtol |b|, atol)), at max_iter, or
 * on a breakdown (sigma <= 0 or NaN: x is the iterate before that step).  No host
 * synchronisation happens inside an iteration: scalars and stop decisions live on
 * the device.  Requires n_rows == n_cols.  b = 0 gives x = 0 after 0 iterations.
 * With SLA_JACOBI in opts->flags the CG is Jacobi-preconditioned; with SLA_BICGSTAB
 * the method is BiCGStab (see the flags above).  A 0 x 0 matrix: every system
 * converges with 0 iterations (d_b and d_x may be NULL; the info records are written,
 * synchronously); a pattern with no entries is A = 0 (SLA_NOT_SPD unless b = 0).
 */
sla_status sla_solve(const sla_csr* A, int64_t batch, const double* d_vals, const double* d_b,
                     double* d_x, const sla_cg_opts* opts, sla_cg_info* d_info, void* stream);

/*
 * sla_solve without any allocation, for callers that cannot allocate device memory
 * during the call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, methods, kernels and results as sla_solve; the
 * solver's workspace (r, p, p', q, and z, d for Jacobi or z for BiCGStab, the
 * reduction partials and the per-system state) lives in a static device array of
 * SLA_NOALLOC_SCRATCH_MIB MiB, which every GPU the library runs on holds until the
 * process ends, instead of memory the handle allocates.  Nothing is allocated by the
 * call: no hipMalloc or hipFree, no registered allocator.  The limit: the workspace must
 * fit the scratch, about 8 x (4 + 2 Jacobi, + 1 BiCGStab) bytes per row and system plus
 * 8 bytes per workgroup and system for the partials: CG up to about 1.5M rows x
 * systems, Jacobi CG and BiCGStab up to about 1M.  A larger problem returns
 * SLA_ERR_INVALID_ARG (the message gives the bytes needed) before any launch.  Other
 * differences from sla_solve, all so that nothing is allocated: batches run the
 * per-system kernels (never the grouped layout), and the plain SpMV reads the 16-bit
 * column offsets only where the handle already holds them (a banded handle builds them
 * on its first plain product; without them the 32-bit columns are read, same row sums).
 * The handle itself (sla_csr_create, and the transpose of a non-symmetric handle)
 * allocates as documented there.  Every call on a GPU shares that GPU's scratch, which
 * keeps the last call's contents (each call initialises what it reads): calls that
 * overlap in time on one GPU, on any streams or threads, race and must not be issued.
 */
#define SLA_NOALLOC_SCRATCH_MIB 50
sla_status sla_solve_noalloc(const sla_csr* A, int64_t batch, const double* d_vals, const double* d_b,
                             double* d_x, const sla_cg_opts* opts, sla_cg_info* d_info, void* stream);

/*
 * Adjoint backward pass of x = A^{-1} b (gist.science summaries, Methodology item 2;
 * paperpeel section 3.2.3): solve A^T lambda = dL/dx with the same method (CG,
 * Jacobi CG or BiCGStab, from opts->flags) and options (threshold relative to
 * |dL/dx|), then
 *   d_gb[b][i]    = lambda_b[i]                       (dL/db)
 *   d_gvals[b][k] = -lambda_b[row(k)] * x_b[col(k)]   (dL/dA on the pattern; nullable)
 *   d_x  [batch][n]  the forward solution (saved by the caller)
 *   d_gx [batch][n]  dL/dx
 * A^T is A for SLA_SYMMETRIC handles, else the transposed pattern with gathered values.
 * Memory: O(n + nnz) per system, whatever the iteration count.
 */
sla_status sla_solve_backward(const sla_csr* A, int64_t batch, const double* d_vals,
                              const double* d_x, const double* d_gx, double* d_gb,
                              double* d_gvals, const sla_cg_opts* opts, sla_cg_info* d_info,
                              void* stream);

/* ------------------------------------------------------------ SparseTensorList */
/*
 * A list of square systems with distinct sparsity patterns, solved together (the
 * pages' second batching mode, SparseTensorList: paperpeel page, section 3.1 "Typed
 * sparse-tensor hierarchy"; gist.science summaries, Methodology item 1).  The items
 * are packed block-diagonally into one pattern, each item's rows starting on a
 * 256-row tile boundary (the rest of its last tile is empty padding), and one grid of
 * workgroups is split among them in proportion to their tiles.  Each item keeps its
 * own scalars, stop test, iteration count and info record, exactly as the systems of
 * a batch do; the arithmetic of every item is that of sla_solve on that item alone
 * (its rows summed in the same order; inner products in a different tree).
 */
typedef struct sla_list sla_list;   /* opaque */

/*
 * Create a list of `items` patterns (1 <= items <= 2^20).  Host arrays [items]:
 *   n[i] >= 1 rows (= columns), nnz[i] >= 0 entries, d_row_ptr[i] / d_col[i] device
 *   pointers to item i's CSR (row_ptr_bits 32 or 64, columns int32 strictly ascending
 *   within a row, in [0, n[i])).
 * Every item is validated on the device (SLA_ERR_INVALID_CSR names the first bad one).
 * The packed pattern and its per-item tables are owned by the list; the caller's
 * arrays are only read during this call.  flags: SLA_SYMMETRIC (every item symmetric)
 * and SLA_EAGER_TRANSPOSE as for sla_csr_create.  Synchronises the stream.
 */
sla_status sla_list_create(sla_list** out, int32_t items, const int64_t* n, const int64_t* nnz,
                           const void* const* d_row_ptr, int32_t row_ptr_bits, const int32_t* const* d_col,
                           uint32_t flags, void* stream);
sla_status sla_list_destroy(sla_list* L);   /* synchronises the device */
/* Packed sizes (rows with padding, entries) and the number of workgroups of the grid. */
sla_status sla_list_info(const sla_list* L, int64_t* n_total, int64_t* nnz_total, int32_t* workgroups);
/* Width in bits of the column indices the list's SpMV reads (16 or 32), as
 * sla_csr_col_bits for the packed pattern. */
sla_status sla_list_col_bits(const sla_list* L, int32_t* col_bits);

/*
 * Solve every item: x_i = A_i^{-1} b_i by CG (or Jacobi CG with SLA_JACOBI; SLA_BICGSTAB
 * is SLA_ERR_UNSUPPORTED here), x0 = 0, the options and stop tests of sla_solve per item.
 *   d_vals[i] [nnz[i]], d_b[i] [n[i]], d_x[i] [n[i]] (outputs): host arrays of device
 *   pointers; d_info device [items].  opts->residual_history, if given, is
 *   [items][max_iter + 1].
 * The values and right-hand sides are copied into packed staging buffers owned by the
 * list, and the solutions copied back.
 */
sla_status sla_list_solve(const sla_list* L, const double* const* d_vals, const double* const* d_b,
                          double* const* d_x, const sla_cg_opts* opts, sla_cg_info* d_info, void* stream);

/*
 * Adjoint backward of sla_list_solve, item by item as sla_solve_backward: A_i^T
 * lambda_i = d_gx[i] (on the packed transpose unless SLA_SYMMETRIC), d_gb[i] = lambda_i,
 * d_gvals[i][k] = -lambda_i[row(k)] x_i[col(k)] (d_gvals nullable; then d_x may be NULL).
 */
sla_status sla_list_solve_backward(const sla_list* L, const double* const* d_vals, const double* const* d_x,
                                   const double* const* d_gx, double* const* d_gb, double* const* d_gvals,
                                   const sla_cg_opts* opts, sla_cg_info* d_info, void* stream);

/* ------------------------------------------------------------------ eigenvalues */
#define SLA_EIG_LARGEST   0   /* the k largest eigenvalues (algebraic), descending */
#define SLA_EIG_SMALLEST  1   /* the k smallest eigenvalues (algebraic), ascending */
#define SLA_EIG_MAX_K     32  /* eigenpairs per call, at most */
#define SLA_EIG_RESTART_MAX_DIM 1024  /* basis size cap when thick restart is on */

typedef struct {
    double tol;                  /* stop when |A u - theta u| <= tol |theta| for every wanted pair (> 0) */
    int64_t max_dim;             /* basis size cap, k <= max_dim <= n (0: min(n, 1000)) */
    int32_t which;               /* SLA_EIG_LARGEST or SLA_EIG_SMALLEST */
    int32_t check_every;         /* Lanczos steps between host checks (0: 16) */
    int64_t max_iter;            /* total Lanczos steps; > max_dim turns on thick restart (0: max_dim) */
    int32_t keep;                /* Ritz vectors kept at a restart, k <= keep < max_dim
                                    (0: min(max_dim - 1, max(k + 1, (max_dim + k) / 2))) */
    int32_t flags;               /* sla_lobpcg: SLA_EIG_JACOBI or 0; sla_eigsh: 0 */
} sla_eig_opts;
#define SLA_EIG_JACOBI 1         /* LOBPCG preconditioned by T = diag(A)^-1 */

typedef struct {
    int64_t iterations;          /* Lanczos steps taken (all bases: restarts included) */
    double max_res;              /* largest residual estimate beta_j |s_r[j]| of the returned pairs */
    int32_t state;               /* SLA_CONVERGED, SLA_MAX_ITER or SLA_BREAKDOWN */
    int32_t restarts;            /* thick restarts taken */
} sla_eig_info;                  /* host struct */

/*
 * k extreme eigenpairs of a symmetric matrix by Lanczos with full reorthogonalization
 * (the pages' .eigsh entry point and its Lanczos eigensolver: paperpeel page, section
 * 3.1 "API"; section 4.3, note to Table 5).  Batch 1.
 *   d_vals   [nnz]   values; the handle must be SLA_SYMMETRIC (else SLA_ERR_UNSUPPORTED)
 *   k        1 <= k <= min(SLA_EIG_MAX_K, max_dim)
 *   d_v0     [n]     start vector (nonzero; the caller draws it, e.g. N(0,1))
 *   d_evals  [k]     output: the Ritz values, from the wanted end
 *   d_evecs  [k][n]  output: unit Ritz vectors, signed so that <u_r, v0> >= 0
 *   info     host output
 * Step j: w = A v_j, alpha_j = <v_j, w>, w -= alpha_j v_j + beta_{j-1} v_{j-1}, then
 * twice w -= V (V^T w) over v_0 .. v_j, beta_j = |w|, v_{j+1} = w / beta_j.  After
 * every step j + 1 >= k the k wanted Ritz pairs (theta_r, s_r) of the tridiagonal
 * T_j are tested: converged when every beta_j |s_r[j]| <= tol |theta_r| (or beta_j =
 * 0: the Krylov space is invariant and the pairs are exact; beta_j counts as 0 when
 * it is at most sqrt(n) eps |T_j|, |T_j| the largest Gershgorin row sum of T_j with
 * beta_j, the rounding level of a reorthogonalized w).  The first step that
 * passes ends the solve (the host checks chunks of steps; the steps past it are
 * discarded).  max_dim steps without convergence: SLA_MAX_ITER with the current Ritz
 * pairs.  An invariant Krylov space of dimension < k: SLA_BREAKDOWN.
 * Thick restart (Wu and Simon, "Thick-restart Lanczos method for large symmetric
 * eigenvalue problems", 2000; the pages name Lanczos without a restart scheme), when
 * max_iter > max_dim: the pairs are tested only when the basis is full (or invariant,
 * or at max_iter steps); if they fail, the keep wanted-end Ritz vectors V s_r and the
 * next Lanczos vector become the new basis (in place, on the device), whose projected
 * matrix is diag(theta_r) bordered by the couplings beta s_r[m-1] (kept on the host,
 * eigenpairs by Householder reduction); the first step of the new basis removes those
 * couplings.  SLA_MAX_ITER after max_iter steps.  Needs max_dim <=
 * SLA_EIG_RESTART_MAX_DIM (SLA_ERR_INVALID_ARG otherwise, and for keep outside
 * [k, max_dim)).
 * Memory: (max_dim + 1) n doubles for the Lanczos vectors, owned by the handle.
 * Synchronises the calling thread with the stream once per chunk of steps.
 */
sla_status sla_eigsh(const sla_csr* A, const double* d_vals, int32_t k, const double* d_v0, double* d_evals,
                     double* d_evecs, const sla_eig_opts* opts, sla_eig_info* info, void* stream);

/*
 * k extreme eigenpairs of a symmetric matrix by LOBPCG, the block eigensolver the pages
 * name beside Lanczos (paperpeel page, section 4.3, note to Table 5; they give no
 * steps).  Knyazev's locally optimal block preconditioned conjugate gradient method
 * (SIAM J. Sci. Comput. 23(2), 2001), unpreconditioned, with an orthonormal
 * Rayleigh-Ritz basis (Hetmaniuk and Lehoucq, J. Comput. Phys. 218, 2006):
 *   X = orth(X0), Rayleigh-Ritz on X; then per iteration R = A X - X diag(theta), the
 *   pairs with |R_r| <= tol |theta_r| are converged (all: SLA_CONVERGED); the others'
 *   residuals W and conjugate directions P are made orthonormal against X (and P
 *   against W) by two projections and Cholesky QR twice on unit-scaled columns (a
 *   block whose Cholesky pivot falls to 1e-14 of the largest is left out of that
 *   iteration); Rayleigh-Ritz on S = [X, W, P] gives the new X = S Y and P = the part
 *   of S Y outside the old X.  A W is the only product with A per iteration.
 *   d_vals   [nnz]   values; the handle must be SLA_SYMMETRIC (else SLA_ERR_UNSUPPORTED)
 *   k        1 <= k <= SLA_EIG_MAX_K, 3 k <= n
 *   d_X0     [k][n]  start block (linearly independent rows, e.g. N(0,1); else
 *                    SLA_ERR_INVALID_ARG)
 *   d_evals  [k]     output: the Ritz values, from the wanted end
 *   d_evecs  [k][n]  output: unit Ritz vectors, signed so that <u_r, X0[r]> >= 0
 *   opts     tol, which, max_iter (iterations; 0: 1000), flags: SLA_EIG_JACOBI applies
 *            Knyazev's preconditioner T = diag(A)^-1 to the residuals (W = T R; every
 *            diagonal entry stored, finite and positive, else SLA_ERR_INVALID_ARG);
 *            max_dim, keep and check_every are not used
 *   info     host output: iterations, max_res (largest |A u - theta u| at the last
 *            test), state (SLA_CONVERGED or SLA_MAX_ITER)
 * Memory: (14 k + 1) n doubles of block vectors, owned by the handle.  Synchronises the
 * calling thread with the stream several times per iteration (the small Gram
 * matrices are factored and solved on the host).
 */
sla_status sla_lobpcg(const sla_csr* A, const double* d_vals, int32_t k, const double* d_X0, double* d_evals,
                      double* d_evecs, const sla_eig_opts* opts, sla_eig_info* info, void* stream);

/*
 * Backward of the eigenvalues of sla_eigsh or sla_lobpcg by the Hellmann-Feynman theorem
 * (dlambda / dA_ij = u_i u_j for a unit eigenvector u: gist.science Japanese summary,
 * Methodology item 2, eigenvalue bullet; paperpeel section 4.3, Eq. (4)): an O(nnz)
 * outer product on the stored entries, no linear solve.
 *   d_evecs  [k][n]  the unit eigenvectors returned by sla_eigsh
 *   d_gevals [k]     dL/dlambda_r
 *   d_gvals  [nnz]   output: dL/dvals[e] = sum_r dL/dlambda_r u_r[row(e)] u_r[col(e)]
 * Only eigenvalue gradients: eigenvector outputs carry none.
 */
sla_status sla_eigsh_backward(const sla_csr* A, int32_t k, const double* d_evecs, const double* d_gevals,
                              double* d_gvals, void* stream);

/*
 * Kernel timing for measurement: while enabled, every kernel the library launches
 * is bracketed by HIP events on its stream; the elapsed times are accumulated per
 * kernel when the enclosing call synchronises (sla_solve / sla_solve_backward with
 * a residual test, or sla_timing_collect).  Disabled by default; enabling it adds
 * event records between launches.
 */
enum {
    SLA_K_CG_INIT = 0,      /* r0 partial norms, x = 0, per-system state reset */
    SLA_K_CG_SPMV = 1,      /* q = A p, partial p^T q (fused schedule: p = r + beta p on the fly, x update) */
    SLA_K_CG_UPDATE = 2,    /* alpha, r -= alpha q, partial r^T r */
    SLA_K_MATVEC = 3,       /* y = A x */
    SLA_K_PATTERN_OUTER = 4,/* gvals = s * u[row] * v[col] */
    SLA_K_GATHER_VALS = 5,  /* transposed values */
    SLA_K_TRANSPOSE = 6,    /* pattern transpose (all its kernels) */
    SLA_K_CG_PUPD = 7,      /* split schedule: step decisions, p = r + beta p, x update */
    SLA_K_GROUP_LAYOUT = 8, /* value layouts: grouped batches (values, x), banded diagonal layout (values) */
    SLA_K_BS_SPMV = 9,      /* BiCGStab: v = A p with <rh, v>, and t = A s with <t, s>, <t, t> */
    SLA_K_BS_VEC = 10,      /* BiCGStab: init, p update, s = r - alpha v, x and r update */
    SLA_K_LZ_SPMV = 11,     /* Lanczos: w = A v_j with <v_j, w> */
    SLA_K_LZ_ORTH = 12,     /* Lanczos: three-term step, reorthogonalization dots and updates, next vector */
    SLA_K_LZ_RITZ = 13,     /* Lanczos: start vector, Ritz vectors, eigenvalue gradient */
    SLA_K_LOB_SPMM = 14,    /* LOBPCG: A W for a block W */
    SLA_K_LOB_GRAM = 15,    /* LOBPCG: Gram products of blocks and their reduction */
    SLA_K_LOB_COMB = 16,    /* LOBPCG: block combinations S Y (projections, Cholesky QR, Ritz vectors) */
    SLA_K_COUNT = 17
};
sla_status sla_timing_enable(int32_t enable);
sla_status sla_timing_reset(void);
sla_status sla_timing_collect(void);    /* synchronises pending timed launches */
sla_status sla_timing_query(int32_t kernel, int64_t* launches, double* total_ms);
/* Algorithmic bytes of the timed launches of a kernel id (each operand column read
 * once, each output written once, the matrix once per product); counted by the LOBPCG
 * block kernels, 0 elsewhere. */
sla_status sla_timing_query_bytes(int32_t kernel, double* bytes);

/* Measurement hook, not part of the solver: one launch of a streaming probe that reads
 * n_read arrays and writes n_write arrays of n doubles (n even, every array 16-byte
 * aligned and holding n doubles), with coalesced 16-byte accesses and nothing else.
 * It measures the bandwidth plain streams of that read/write mix reach, the ceiling
 * beside which the CG kernels' bandwidth is reported.  Supported mixes (n_read,
 * n_write): (1,0) read, (0,1) write, (1,1) copy, (2,1) triad (the CG update's mix),
 * (10,3) about the banded CG SpMV's 78 bytes read per 24 written.  in / out: host
 * arrays of device pointers.  unroll 1, 2 or 4 (16-byte accesses in flight per thread
 * and array), nontemporal 0/1 (the streaming hint on every access), blocks_per_cu in
 * [1, 8] (grid = CUs x blocks_per_cu).  part: device array of at least 8 x CUs doubles,
 * written by read-only probes (n_write == 0) with per-workgroup sums; may be NULL
 * otherwise.  Enqueued on `stream`; returns SLA_ERR_INVALID_ARG or SLA_ERR_UNSUPPORTED
 * (another mix or unroll) before any launch. */
sla_status sla_probe_stream(int32_t n_read, int32_t n_write, const double* const* in, double* const* out,
                            int64_t n, int32_t unroll, int32_t nontemporal, int32_t blocks_per_cu,
                            double* part, void* stream);

const char* sla_status_string(sla_status s);
const char* sla_last_error(void);
int32_t sla_version(void);             /* 100 * major + minor */

#ifdef __cplusplus
}
#endif
#endif /* SLA_H */
