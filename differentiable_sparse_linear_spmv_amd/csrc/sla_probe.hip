// sla_probe.hip -- streaming bandwidth probes, a measurement hook beside the solver.
//
// Each probe kernel reads NR arrays and writes NW arrays of n doubles with fully
// coalesced 16-byte accesses, nothing else: the rate plain streams of that read/write
// mix reach on this GPU.  The solver never calls them.  They give the measured ceiling
// that the CG kernels' bandwidth is set beside (an HBM-bound CG iteration moves a fixed
// mix of reads and writes, about 3.3 bytes read per byte written in the SpMV and 2 in
// the update).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sla.h"
#include "sla_internal.h"

namespace sla {
namespace {

constexpr int kProbeMaxIn = 12;
constexpr int kProbeMaxOut = 4;

struct ProbeArgs {
    const double2* in[kProbeMaxIn];
    double2* out[kProbeMaxOut];
    double* part;    // [gridDim.x]: read-only probes keep their sums (no dead loads)
    int64_t n2;      // elements of double2 per array
};

template <bool NT>
__device__ __forceinline__ double2 ld2(const double2* p)
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
__device__ __forceinline__ void st2(double2* p, double2 v)
{
    if constexpr (NT) {
        __builtin_nontemporal_store(v.x, &p->x);
        __builtin_nontemporal_store(v.y, &p->y);
    } else {
        *p = v;
    }
}

// Grid-stride over trips of U * kBlock double2 per array; within a trip thread t takes
// elements t, t + kBlock, ... so every wave's access is one contiguous 1 KiB run.
template <int NR, int NW, int U, bool NT>
__global__ __launch_bounds__(kBlock) void k_probe(ProbeArgs a)
{
    const int tid = threadIdx.x;
    const int64_t trip = static_cast<int64_t>(U) * kBlock;
    double acc = 0.0;
    for (int64_t b0 = static_cast<int64_t>(blockIdx.x) * trip; b0 < a.n2; b0 += trip * gridDim.x) {
        const bool full = b0 + trip <= a.n2;
        double2 v[NR > 0 ? NR : 1][U];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = b0 + u * kBlock + tid;
                v[r][u] = (full || i < a.n2) ? ld2<NT>(a.in[r] + i) : double2{0.0, 0.0};
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            double sx = 1.0, sy = 2.0;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                sx = sx + v[r][u].x;
                sy = sy + v[r][u].y;
            }
            const int64_t i = b0 + u * kBlock + tid;
            if constexpr (NW == 0) {
                acc = acc + (sx + sy);
            } else if (full || i < a.n2) {
#pragma unroll
                for (int w = 0; w < NW; ++w) st2<NT>(a.out[w] + i, double2{sx + w, sy - w});
            }
        }
    }
    if constexpr (NW == 0) {
        __shared__ double s_red[kBlock / 64];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc = acc + __shfl_xor(acc, off, 64);
        if ((tid & 63) == 0) s_red[tid >> 6] = acc;
        __syncthreads();
        if (tid == 0) a.part[blockIdx.x] = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    }
}

using ProbeKernel = void (*)(ProbeArgs);

template <int NR, int NW>
ProbeKernel probe_kernel(int unroll, bool nt)
{
    switch (unroll) {
    case 1: return nt ? k_probe<NR, NW, 1, true> : k_probe<NR, NW, 1, false>;
    case 2: return nt ? k_probe<NR, NW, 2, true> : k_probe<NR, NW, 2, false>;
    case 4: return nt ? k_probe<NR, NW, 4, true> : k_probe<NR, NW, 4, false>;
    default: return nullptr;
    }
}

ProbeKernel pick(int nr, int nw, int unroll, bool nt)
{
    if (nr == 1 && nw == 0) return probe_kernel<1, 0>(unroll, nt);
    if (nr == 0 && nw == 1) return probe_kernel<0, 1>(unroll, nt);
    if (nr == 1 && nw == 1) return probe_kernel<1, 1>(unroll, nt);
    if (nr == 2 && nw == 1) return probe_kernel<2, 1>(unroll, nt);
    if (nr == 10 && nw == 3) return probe_kernel<10, 3>(unroll, nt);
    return nullptr;
}

}  // namespace
}  // namespace sla

extern "C" sla_status sla_probe_stream(int32_t n_read, int32_t n_write, const double* const* in, double* const* out,
                                       int64_t n, int32_t unroll, int32_t nontemporal, int32_t blocks_per_cu,
                                       double* part, void* stream)
{
    using namespace sla;
    if (n < 2 || (n & 1) || n_read < 0 || n_write < 0 || n_read > kProbeMaxIn || n_write > kProbeMaxOut ||
        blocks_per_cu < 1 || blocks_per_cu > 8)
        return SLA_ERR_INVALID_ARG;
    if ((n_read > 0 && !in) || (n_write > 0 && !out) || (n_write == 0 && !part)) return SLA_ERR_INVALID_ARG;
    ProbeKernel k = pick(n_read, n_write, unroll, nontemporal != 0);
    if (!k) return SLA_ERR_UNSUPPORTED;
    ProbeArgs a{};
    for (int r = 0; r < n_read; ++r) {
        if (!in[r] || (reinterpret_cast<uintptr_t>(in[r]) & 15)) return SLA_ERR_INVALID_ARG;
        a.in[r] = reinterpret_cast<const double2*>(in[r]);
    }
    for (int w = 0; w < n_write; ++w) {
        if (!out[w] || (reinterpret_cast<uintptr_t>(out[w]) & 15)) return SLA_ERR_INVALID_ARG;
        a.out[w] = reinterpret_cast<double2*>(out[w]);
    }
    a.part = part;
    a.n2 = n / 2;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return SLA_ERR_HIP;
    const int64_t trips = (a.n2 + int64_t(unroll) * kBlock - 1) / (int64_t(unroll) * kBlock);
    int64_t g = static_cast<int64_t>(ncu) * blocks_per_cu;
    if (g > trips) g = trips;
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(g)), dim3(kBlock), 0, static_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? SLA_OK : SLA_ERR_HIP;
}
