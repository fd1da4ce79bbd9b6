// sla_internal.h -- shared declarations between the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sla.h"

namespace sla {

constexpr int kBlock = 256;   // threads per workgroup (4 waves of 64)
constexpr int kTile = 256;    // CSR rows per tile: one row per lane

// LDS capacities (stored entries per tile) of the staged SpMV variants.  The
// handle picks the smallest that holds its largest tile; tiles above the cap
// take the wave-per-row path inside the same kernel.
constexpr int kCapSmall = 1280;   // 5 entries per row
constexpr int kCapMid = 2048;     // 8 per row
constexpr int kCapLarge = 4096;   // 16 per row
// Patterns with a row of more than kBinLaneMax entries take the products-first variant
// of the staged kernels (LDS of kCapLarge entries): every entry's product is formed in
// parallel over the workgroup into LDS, then each lane sums its row's products in order.
constexpr int kBinLaneMax = 32;
constexpr int kCapSkew = kCapLarge + 1;

// Banded patterns (every entry within kBandHalo of the diagonal or of distance S from
// it) take the line-walking SpMV; its segments extend kBandHalo past each strip end.
constexpr int kBandHalo = 8;
// Lines per block of work of the banded SpMV, at most (each block starts its LDS ring
// afresh, reading two segments more than it uses: 1/16 more operand reads at 32 lines).
constexpr int kBandBlockLines = 32;
// Resident workgroups per CU of the banded SpMV when one SpMV streams more than
// kBandStreamBytes: with few workgroups sweeping one front, HBM sees the longest
// sequential runs (measured on 169M rows: 2 per CU beat 1 and 4).  Smaller systems,
// served largely from the 256 MB Infinity Cache, run at full occupancy.
constexpr int kBandBlocksPerCu = 2;
// The same for the diagonal-layout SpMV (k_cg_spmv_dia): one workgroup per CU (169M
// rows: 2879 us per launch, against 2997 us with 2, 3050 with 3 and 3058 with 4).
constexpr int kDiaBlocksPerCu = 1;
constexpr int64_t kBandStreamBytes = int64_t(1) << 30;

// Patterns that are not banded but reach columns at least this far from the diagonal
// gather from all over the operand: they take the split CG schedule (p_k formed by its
// own pass, then gathered alone), which halves the gathers' cache requests.
constexpr int64_t kSplitMinSpan = 4096;

// Grouped batches: systems interleaved per element in groups of kGroup (a 32-byte
// piece per gathered element).  Batches of at least kGroupMinBatch systems, a
// multiple of kGroup, on split-schedule patterns use the grouped kernels.
constexpr int kGroup = 4;
constexpr int kGroupMinBatch = 8;
// Entries per 64-row tile staged by the grouped SpMV: rows of at most 8 or 16 entries.
constexpr int kGCapSmall = 512;
constexpr int kGCapLarge = 1024;
// The grouped SpMV keeps the operand in an LDS window when the (reordered) pattern's
// bandwidth is at most this many rows (7 chunks of 64 rows on each side of a tile).
constexpr int kGWinMaxHalo = 448;

// Per-system solver state in device memory (80 bytes).  Double-buffered by the
// parity of the iteration index so that a kernel reads the previous value while
// its first workgroup writes the new one.
struct SysState {
    int64_t stop_iter;   // INT64_MAX while running; else the iteration at which it stopped
                         // (BiCGStab: the phase 5 k + position of the kernel that stopped it)
    double rho[2];       // rho_k = r_k^T r_k (Jacobi r_k^T z_k, BiCGStab rh^T r_k), slot k & 1
    double alpha[2];     // alpha_k, slot k & 1
    double thr;          // stop threshold max(rtol |rhs|, atol)
    double rhs;          // |rhs|
    double rr;           // Jacobi, BiCGStab: |r_k|^2 of the last step (rho holds another product)
    double omega[2];     // BiCGStab: omega_k, slot k & 1
};
static_assert(sizeof(SysState) == 80, "SysState layout");

// Arguments of the fused CG kernels (passed by value).
struct CgArgs {
    const void* row_ptr;     // int32 or int64 [n + 1]
    const int32_t* col;      // [nnz]
    const int16_t* col16;    // nullable, [nnz]: col minus the tile's first row (staged SpMV)
    const double* vals;      // [batch][nnz]
    const double* b;         // [batch][n]   right-hand side (r_0)
    double* x;               // [batch][n]
    double* r;               // [batch][n]
    double* p0;              // [batch][n]   p_k for even k
    double* p1;              // [batch][n]   p_k for odd k
    double* q;               // [batch][n]   A p_k
    double* part_sigma;      // [batch][G]   written by k_cg_spmv
    double* part_rho;        // [batch][Gu]  written by k_cg_init / k_cg_update (rho_k partials)
    double* part_rr;         // [batch][Gu]  Jacobi: r^T r partials (the stop test)
    double* part_aux;        // [batch][Gu]  Jacobi: bad-diagonal flags of k_cg_init; BiCGStab: s^T s
    double* part_tt;         // [batch][G]   BiCGStab: t^T t (t = A s), written by the SpMV
    double* z;               // [batch][n]   Jacobi: z_k = M^{-1} r_k
    double* dg;              // [batch][n]   Jacobi: the diagonal of A
    SysState* st;            // [batch]
    sla_cg_info* info;       // [batch]
    double* hist;            // nullable, [batch][max_iter + 1]
    int32_t* n_active;       // systems still running
    int64_t n;
    int64_t nnz;
    int64_t ntiles;
    int64_t max_iter;
    double rtol;
    double atol;
    int32_t fixed;
    int32_t G;               // workgroups per system of k_cg_spmv
    int32_t Gu;              // workgroups per system of k_cg_init and k_cg_update
    int32_t batch;
    int32_t xcd_remap;       // 1: map workgroups so each XCD streams contiguous tiles
    int32_t sys_per_xcd;     // 1: batch % 8 == 0; every system runs on one XCD
    int32_t split;           // 1: split schedule (k_cg_pupd forms p_k, the SpMV gathers it)
    int32_t jacobi;          // 1: Jacobi-preconditioned CG
    int32_t stream_nt;       // 1: the update kernel streams with the non-temporal hint
    int32_t groups;          // grouped batch: number of groups (r, p0, p1, q, vals, xg grouped)
    int32_t cap;             // grouped batch: entries per tile staged (kGCapSmall or kGCapLarge)
    double* xg;              // grouped batch: x in the grouped layout
    int32_t g_halo;          // grouped batch: operand window halo (rows, a multiple of 64), 0 = no window
    const int16_t* g_col16;  // grouped batch with a window: columns minus the first row of their 64-row tile
    const int32_t* gperm;    // grouped batch on a reordered pattern: row i is the caller's row gperm[i]
    // SparseTensorList (distinct patterns, packed block-diagonally; null otherwise):
    // system s owns tiles [list_tiles[s], list_tiles[s + 1]) and workgroups
    // [list_wg[s], list_wg[s + 1]) of a one-dimensional grid (the same for every kernel);
    // its real rows end at list_rend[s] (the rest of its last tile is padding).
    const int32_t* list_wg;
    const int64_t* list_tiles;
    const int64_t* list_rend;
    int32_t list_items;
    int32_t band_block;      // banded SpMV: lines per block of work
    int64_t band_stride;     // banded SpMV: line length S (0: plain SpMV)
    int64_t band_lines;      // banded SpMV: ceil(n / S)
    int32_t wide_update;     // 1: k_cg_update_wide (16-byte accesses, grid-stride row pairs)
    // Diagonal layout of a banded pattern (k_cg_spmv_dia; dia_nd = 0: not used).  The
    // pattern's distinct offsets c - i, ascending, are b S + e with b in {-1, 0, 1} and
    // |e| <= kBandHalo; diagonal d lives in LDS ring segment dia_b[d] + 1 (line l - 1, l,
    // l + 1) at position dia_e[d] + kBandHalo + (the row's position in the strip).
    const double* dia_vals;  // [batch][dia_nd][n]: value of row i on diagonal d at [d][i]
    const double* dia_v[16]; // system 0's diagonal d at dia_v[d] (d < dia_nd; the last one repeated after)
    const void* dia_mask;    // [n] uint8 (dia_nd <= 8) or uint16: bit d set if row i stores diagonal d
    int32_t dia_nd;
    int32_t dia_shift;       // diagonal layout: 8 when windows of odd lines are shifted onto 128-byte boundaries
    int8_t dia_b[16];
    int8_t dia_e[16];
};

// Diagonal layout of banded patterns: offsets c - i = b S + e (b in {-1, 0, 1}, |e| <=
// kBandHalo) numbered by code (b + 1) kDiaCodesPerBand + e + kBandHalo, ascending in c - i.
constexpr int kDiaMax = 16;                       // diagonals of the layout, at most
constexpr int kDiaCodesPerBand = 2 * kBandHalo + 1;   // e in [-kBandHalo, kBandHalo]
constexpr int kDiaCodes = 3 * kDiaCodesPerBand;   // 51
struct DiaMap {
    int8_t d_of_code[kDiaCodes + 1];   // diagonal index of each code, -1 if the pattern has none
};
// Codes present in a banded pattern of line stride S (rows with 32-bit row pointers):
// out[0] |= bits of codes 0..31, out[1] |= bits of codes 32..50; out[2] != 0 if some
// entry has no code (not banded with stride S).  out zeroed by the caller.
hipError_t launch_dia_codes(const int32_t* rp, const int32_t* col, int64_t n, int32_t S, uint32_t* out,
                            hipStream_t s);
// mask[i] (uint8 when m16 is false, else uint16): bit d set if row i stores diagonal d.
hipError_t launch_dia_mask(const int32_t* rp, const int32_t* col, int64_t n, int32_t S, const DiaMap& m, void* mask,
                           bool m16, hipStream_t s);
// out[b][d][i] = vals[b][k] for every stored entry k = (i, c) of diagonal d (entries a row
// does not store are left as they are: the mask excludes them).
hipError_t launch_dia_vals(const int32_t* rp, const int32_t* col, const double* vals, int64_t n, int64_t nnz, int32_t S,
                           const DiaMap& m, int nd, int batch, double* out, hipStream_t s);
int cg_dia_blocks_per_cu(int nd);   // the diagonal-layout SpMV

// Lanczos eigensolver (sla_eigsh).  V [max_dim + 1][n]: row j is the Lanczos vector
// v_j; w [n] the vector being orthogonalized.  Grids: Gu workgroups for the streaming
// kernels, Gd for the reorthogonalization dots (kLzRows rows each), G for the SpMV.
constexpr int kLzRows = 1024;      // rows per workgroup of the reorthogonalization dots
constexpr int kEigMaxK = 32;       // eigenpairs per call, at most
constexpr int64_t kEigRestartMaxDim = 1024;   // basis size cap with thick restart
struct LzArgs {
    double* V;
    double* w;
    const double* v0;        // start vector (caller's)
    double* part;            // [Gu] norm partials
    double* part_h;          // [max_dim + 1][Gd] reorthogonalization dot partials
    double* h;               // [max_dim + 1] reorthogonalization coefficients
    double* alpha;           // [max_dim] diagonal of T
    double* beta;            // [max_dim] off-diagonal of T (beta_j = |w| after step j)
    const double* part_sigma;// [G] the SpMV's partials of <v_j, A v_j>
    const double* S;         // [k][m] Ritz coefficients (row r: eigenvector r of T)
    double* U;               // [k][n] Ritz vectors
    const double* scale;     // [k] signed norms of the Ritz vectors (u_r is divided by it)
    double* part_ritz;       // [2 k][Gu] partials of <u_r, u_r> and <u_r, v_0>
    int64_t n;
    int64_t m;               // Ritz vectors: Krylov dimension
    int32_t G, Gu, Gd;
    int32_t k;
};
// which: 0 |v0|^2 partials, 1 v_0 = v0 / nrm, 2 three-term step of column j (alpha_j from
// the SpMV partials), 3 dots of w with columns 0 .. j, 4 their reduction into h, 5 w -=
// V h (last: with |w|^2 partials), 6 beta_j and v_{j+1}, 7 Ritz vectors with partials,
// 8 division of the Ritz vectors by their signed norms.
hipError_t launch_lz(int which, const LzArgs& a, int64_t j, double nrm, int last, hipStream_t s);
// Thick restart in place: V[r] = sum_{l<m} S[r][l] V[l] for r < lk (S [lk][m] on the
// device), then V[lk] = V[m].  Needs 1 <= lk < m <= kLzStage.
constexpr int64_t kLzStage = 8192;   // doubles of V staged in LDS per workgroup (64 KiB)
// The first reorthogonalization pass's update fused with the second pass's dots (one
// read of V instead of two) for bases of at most kLzFusedCols columns.
constexpr int kLzFusedCols = 32;
hipError_t launch_lz_axpy_dots(const LzArgs& a, int64_t ncols, hipStream_t s);
hipError_t launch_lz_restart(const LzArgs& a, int64_t m, int64_t lk, hipStream_t s);
// dL/dvals[e] = sum_r g[r] U[r][row(e)] U[r][col(e)] (Hellmann-Feynman), g and U on the device.
hipError_t launch_eig_grad(const void* row_ptr, int rp_bits, const int32_t* col, const double* U, const double* g,
                           int k, int64_t n, int64_t nnz, double* gvals, hipStream_t s);

// Block kernels (LOBPCG).  A block is a set of n-vectors, column c at base + c n, named
// by device index lists; coefficient matrices are device arrays.
constexpr int kBlkMaxCols = 96;      // columns of a Gram operand (3 x SLA_EIG_MAX_K)
constexpr int kBlkGramGroups = 1024; // workgroups of a Gram product, at most (partials per pair)
// out[idx_out[c]] = A in[idx_in[c]], c < q <= kBlkMaxCols.
hipError_t launch_blk_spmm(const void* rp, int rp_bits, const int32_t* col, const double* vals, const double* in,
                           const int32_t* idx_in, double* out, const int32_t* idx_out, int q, int64_t n,
                           hipStream_t s);
// out[a mv + b] = <A[ia[a]], B[ib[b]]> (a < mu, b < mv, both <= kBlkMaxCols), summed in
// a fixed order; part: blk_gram_groups(n) * mu * mv doubles of scratch (at most).  same:
// B's columns are A's (mu == mv; B and ib are not read), which are then loaded once.
// yproj (mu >= mv): instead of out, the coefficients [I; -out] [(mv + mu)][mv] of the
// projection Z - B (B^T Z) over [Z, B] (A = B, the orthonormal block; B = Z).
int blk_gram_groups(int64_t n);
hipError_t launch_blk_gram(const double* A, const int32_t* ia, int mu, const double* B, const int32_t* ib, int mv,
                           int64_t n, double* part, double* out, hipStream_t s, bool same = false,
                           double* yproj = nullptr);
// out[idx_out[c]] = sum_j Y[j][c] in[idx_in[j]] (c < q <= 32, Y [m][q]); part (nullable):
// blk_comb_groups(n) * q partials of |out[c]|^2, [group][c].  out must not alias in.
int blk_comb_groups(int64_t n);
// out[p] = sum over g < G of part[g][p] (g ascending), p < np.
hipError_t launch_blk_reduce(const double* part, int G, int np, double* out, hipStream_t s);
// tinv[i] = 1 / a_ii; part[g] (blk_comb_groups(n) doubles): rows of group g whose a_ii
// is missing, not finite or not positive (tinv 0 there).
hipError_t launch_blk_diag_inv(const void* rp, int rp_bits, const int32_t* col, const double* vals, int64_t n,
                               double* tinv, double* part, hipStream_t s);
// T [w][w] (w <= SLA_EIG_MAX_K): the Cholesky QR coefficients of the block Z = A[ia[c]]
// (c < w) from its Gram matrix (left in gram, w w doubles), Z T orthonormal; scale: unit
// columns first.  part: scratch as for launch_blk_gram.  flag (device-visible): set with
// scale, read otherwise; a failed block gets T = 0 and flag 0.
hipError_t launch_blk_gram_orth(const double* A, const int32_t* ia, int w, int64_t n, double* part, double* gram,
                                bool scale, double pivot, double* flag, double* T, hipStream_t s);
// out[idx_out[c]] = sum_{j < m} Y[j][c] in[idx_in[j]] and out[idx_out2[c]] = the same sum
// from j = j0, in one pass (c < q <= 32, Y [m][q]); n even, in and out 16-byte aligned.
hipError_t launch_blk_comb_dual(const double* in, const int32_t* idx_in, int m, int j0, const double* Y,
                                double* out, const int32_t* idx_out, const int32_t* idx_out2, int q, int64_t n,
                                hipStream_t s);
// out[idx_out[c]][i] = in[idx_in[c]][i] * t[i], c < q.
hipError_t launch_blk_rowscale(const double* in, const int32_t* idx_in, double* out, const int32_t* idx_out, int q,
                               int64_t n, const double* t, hipStream_t s);
hipError_t launch_blk_comb(const double* in, const int32_t* idx_in, int m, const double* Y, double* out,
                           const int32_t* idx_out, int q, int64_t n, double* part, hipStream_t s,
                           bool pairs = false);

// Bandwidth-reducing order of a square pattern (reverse Cuthill-McKee, host code,
// sla_reorder.hip): perm[new] = old.  rp / col are host copies of the pattern.
void rcm_order(const int32_t* rp, const int32_t* col, int64_t n, int32_t* perm);

// Wanted eigenpairs of a symmetric tridiagonal matrix (host code, sla_tridiag.hip):
// diagonal a[0..m), off-diagonal b[0..m-1).  The k largest (descending) or smallest
// (ascending) eigenvalues into theta[k], unit eigenvectors into S[k][m].
void tridiag_eigpairs(const double* a, const double* b, int m, int k, bool largest, double* theta, double* S);
// The same for a dense symmetric H [m][m] (row-major): Householder reduction to
// tridiagonal form, then tridiag_eigpairs, then the back-transform.
void sym_eigpairs(const double* H, int m, int k, bool largest, double* theta, double* S);

// Optional timing events for the next single-kernel launch: when set, launchers use
// hipExtLaunchKernelGGL so the events carry the kernel's own start and end times.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchEvents& launch_events();

// Resident workgroups per CU of the SpMV kernel variant for this pattern (its grid is
// sized to fill the GPU exactly once).
int cg_blocks_per_cu(int rp_bits, int cap, int64_t n, bool split);
int cg_band_blocks_per_cu(int cap);   // the banded SpMV (32-bit row pointers only)
int cg_group_blocks_per_cu(int cap, bool win);   // the grouped SpMV (win: the windowed variant)

// Host-side launchers (defined in sla_kernels.hip).  All return hipError_t of the launch.
hipError_t launch_cg_init(const CgArgs& a, hipStream_t s);
hipError_t launch_cg_diag(const CgArgs& a, int rp_bits, hipStream_t s);   // Jacobi: diagonal, before init
hipError_t launch_cg_spmv(const CgArgs& a, int64_t k, int rp_bits, int cap, hipStream_t s);
hipError_t launch_cg_update(const CgArgs& a, int64_t k, hipStream_t s);
hipError_t launch_cg_pupd(const CgArgs& a, int64_t k, hipStream_t s);   // split schedule
// Grouped batch: values into the grouped layout, and the CG kernels
// (which: 0 init, 1 p update, 2 SpMV, 3 update, 4 x back to the caller's layout,
// 5 the Jacobi diagonal in the grouped layout).
// eperm (nullable): entry k of the reordered pattern is entry eperm[k] of the caller's.
hipError_t launch_group_vals(const double* vals, double* out, int64_t nnz, int groups, const int32_t* eperm,
                             hipStream_t s);
hipError_t launch_gcg(int which, const CgArgs& a, int64_t k, hipStream_t s);
// BiCGStab (which: 0 init, 1 p update, 2 v = A p, 3 s, 4 t = A s, 5 update).  Vectors:
// r in a.r, p in a.p0, v in a.q, s in a.p1, t in a.z; rh = b.
hipError_t launch_bs(int which, const CgArgs& a, int64_t k, int rp_bits, int cap, hipStream_t s);
int bs_blocks_per_cu(int rp_bits, int cap, int64_t n);   // the BiCGStab SpMV (t = A s variant)

// SparseTensorList packing: item pattern (row_ptr of rp_bits, col) with n rows and nnz
// entries into the packed pattern at row r0 and entry e0, its rows padded with empty
// rows up to r0 + rows_padded; columns shifted by r0.  out_rp has the packed width.
hipError_t launch_pack_pattern(const void* rp, int rp_bits, const int32_t* col, int64_t n, int64_t nnz, int64_t r0,
                               int64_t e0, int64_t rows_padded, void* out_rp, int out_bits, int32_t* out_col,
                               hipStream_t s);

hipError_t launch_matvec(const void* row_ptr, int rp_bits, const int32_t* col, const double* vals,
                         const double* x, double* y, int64_t n_rows, int64_t nnz, int64_t n_cols,
                         int batch, int cap, hipStream_t s);

hipError_t launch_pattern_outer(const void* row_ptr, int rp_bits, const int32_t* col, double sign,
                                const double* u, int64_t u_stride, const double* v,
                                int64_t v_stride, double* g, int64_t n_rows, int64_t nnz,
                                int batch, hipStream_t s);

hipError_t launch_gather_vals(const int64_t* perm, const double* vals, double* out, int64_t nnz,
                              int batch, hipStream_t s);

// CSR checks and pattern analysis.  out[kChkCount] on entry: {0, 0, 0, INT32_MAX, 0}.
// out[kChkErr] gets a nonzero code ORed in on any problem; out[kChkTileMax] the most
// entries of any 256-row tile; out[kChkRowMax] the most entries of any row;
// out[kChkFarMin] / out[kChkFarMax] the least / largest |c - i| over the entries with
// |c - i| > kBandHalo (the band analysis).
constexpr int kChkErr = 0, kChkTileMax = 1, kChkRowMax = 2, kChkFarMin = 3, kChkFarMax = 4, kChkCount = 5;
hipError_t launch_validate(const void* row_ptr, int rp_bits, const int32_t* col, int64_t n_rows,
                           int64_t n_cols, int64_t nnz, int32_t* out, hipStream_t s);

// out[i] = (int32) in[i] for i < n: 32-bit copy of 64-bit row pointers whose values fit.
hipError_t launch_narrow_rp(const int64_t* in, int32_t* out, int64_t n, hipStream_t s);

// 16-bit column offsets for the staged CG SpMV: out[e] = col[e] - (first row of the
// 256-row tile holding entry e).  They fit when every stored entry has
// |c - i| <= kCol16MaxSpan (then c - row0 lies in [-kCol16MaxSpan, 32767]).
constexpr int32_t kCol16MaxSpan = 32767 - (kTile - 1);
hipError_t launch_col16(const int32_t* rp, const int32_t* col, int16_t* out, int64_t n_rows, hipStream_t s);
// The same for the banded SpMV (line stride S <= kCol16MaxSpan): offsets from the
// first row of the window (line i / S, strip (i % S) / kTile) that holds row i.
hipError_t launch_colb16(const int32_t* rp, const int32_t* col, int16_t* out, int64_t n_rows, int32_t S,
                         hipStream_t s);

// Transposed pattern: row_ptr_t (same width as rp_bits) [n_cols + 1], col_t [nnz],
// perm [nnz] (position in A of each entry of A^T).  scratch: see transpose_scratch_bytes.
size_t transpose_scratch_bytes(int64_t n_rows, int64_t n_cols, int64_t nnz);
hipError_t launch_transpose(const void* row_ptr, int rp_bits, const int32_t* col, int64_t n_rows,
                            int64_t n_cols, int64_t nnz, void* row_ptr_t, int32_t* col_t,
                            int64_t* perm, void* scratch, hipStream_t s);

}  // namespace sla
