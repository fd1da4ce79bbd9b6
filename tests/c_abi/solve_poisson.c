/*
 * A C consumer of the library, no Python: the 5-point Poisson matrix on an N x N grid
 * (the pages' 2-D Poisson workload, torch-sla, paperpeel page, section 4.1) is built
 * on the host, solved by sla_solve to rtol 1e-10 and differentiated by
 * sla_solve_backward for L = 0.5 |x|^2; the host then checks the true residual
 * |b - A x| / |b| <= 1e-9, both solves converged, and dL/dvals[e] = -lambda[row(e)]
 * x[col(e)] on every stored entry, to the bit (one rounded product, as the library).
 * Exit status 0 on success.  Usage: solve_poisson [N]
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "sla.h"

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
            return 2;                                                             \
        }                                                                         \
    } while (0)
#define CHECK_SLA(x)                                                              \
    do {                                                                          \
        sla_status s_ = (x);                                                      \
        if (s_ != SLA_OK) {                                                       \
            fprintf(stderr, "%s: %s (%s)\n", #x, sla_status_string(s_), sla_last_error()); \
            return 3;                                                             \
        }                                                                         \
    } while (0)

int main(int argc, char** argv)
{
    const int N = argc > 1 ? atoi(argv[1]) : 96;
    const int n = N * N;
    const int nnz = 5 * n - 4 * N;
    int32_t* rp = malloc(sizeof(int32_t) * (n + 1));
    int32_t* col = malloc(sizeof(int32_t) * nnz);
    double* val = malloc(sizeof(double) * nnz);
    double *b = malloc(sizeof(double) * n), *x = malloc(sizeof(double) * n);
    double *lam = malloc(sizeof(double) * n), *gv = malloc(sizeof(double) * nnz);
    int k = 0;
    for (int i = 0; i < n; ++i) {   /* row i = (r, c): neighbours in ascending column order */
        const int r = i / N, c = i % N;
        rp[i] = k;
        if (r > 0) { col[k] = i - N; val[k++] = -1.0; }
        if (c > 0) { col[k] = i - 1; val[k++] = -1.0; }
        col[k] = i; val[k++] = 4.0;
        if (c < N - 1) { col[k] = i + 1; val[k++] = -1.0; }
        if (r < N - 1) { col[k] = i + N; val[k++] = -1.0; }
        b[i] = sin(0.37 * i) + 0.5;
    }
    rp[n] = k;
    if (k != nnz) return 4;

    int32_t *d_rp, *d_col;
    double *d_val, *d_b, *d_x, *d_lam, *d_gv;
    sla_cg_info *d_info, info[2];
    CHECK_HIP(hipMalloc((void**)&d_rp, sizeof(int32_t) * (n + 1)));
    CHECK_HIP(hipMalloc((void**)&d_col, sizeof(int32_t) * nnz));
    CHECK_HIP(hipMalloc((void**)&d_val, sizeof(double) * nnz));
    CHECK_HIP(hipMalloc((void**)&d_b, sizeof(double) * n));
    CHECK_HIP(hipMalloc((void**)&d_x, sizeof(double) * n));
    CHECK_HIP(hipMalloc((void**)&d_lam, sizeof(double) * n));
    CHECK_HIP(hipMalloc((void**)&d_gv, sizeof(double) * nnz));
    CHECK_HIP(hipMalloc((void**)&d_info, sizeof(sla_cg_info) * 2));
    CHECK_HIP(hipMemcpy(d_rp, rp, sizeof(int32_t) * (n + 1), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_col, col, sizeof(int32_t) * nnz, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_val, val, sizeof(double) * nnz, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_b, b, sizeof(double) * n, hipMemcpyHostToDevice));

    sla_csr* A = NULL;
    CHECK_SLA(sla_csr_create(&A, n, n, nnz, d_rp, 32, d_col, SLA_SYMMETRIC, NULL));
    sla_cg_opts o = {1e-10, 0.0, 100000, 0, 0u, NULL};
    CHECK_SLA(sla_solve(A, 1, d_val, d_b, d_x, &o, d_info, NULL));
    /* L = 0.5 |x|^2: dL/dx = x */
    CHECK_SLA(sla_solve_backward(A, 1, d_val, d_x, d_x, d_lam, d_gv, &o, d_info + 1, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(x, d_x, sizeof(double) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lam, d_lam, sizeof(double) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gv, d_gv, sizeof(double) * nnz, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(info, d_info, sizeof(info), hipMemcpyDeviceToHost));

    double rr = 0.0, bb = 0.0;
    int grad_bad = 0;
    for (int i = 0; i < n; ++i) {
        double ax = 0.0;
        for (int e = rp[i]; e < rp[i + 1]; ++e) {
            ax += val[e] * x[col[e]];
            const double want = -lam[i] * x[col[e]];
            if (gv[e] != want) ++grad_bad;
        }
        const double ri = b[i] - ax;
        rr += ri * ri;
        bb += b[i] * b[i];
    }
    const double res = sqrt(rr / bb);
    printf("N=%d n=%d iterations %lld + %lld, states %d %d, true residual %.3e, gradient entries off %d\n", N,
           n, (long long)info[0].iterations, (long long)info[1].iterations, info[0].state, info[1].state, res,
           grad_bad);
    sla_csr_destroy(A);
    hipFree(d_rp); hipFree(d_col); hipFree(d_val); hipFree(d_b); hipFree(d_x); hipFree(d_lam); hipFree(d_gv);
    hipFree(d_info);
    const int ok = info[0].state == SLA_CONVERGED && info[1].state == SLA_CONVERGED && res <= 1e-9 &&
                   grad_bad == 0;
    return ok ? 0 : 1;
}
