// kda_validate.hip -- debug checks: the value domains the KDA kernels assume
// (kda_validate_inputs) and the workgroup placement the fused launches assume
// (kda_workgroup_xcds).
//
// Domains: page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section 3.3,
// lower-bounded decay: the log-decay g lies in [g_min, 0] with g_min = -5, which is
// what keeps every decay factor of a 16-position tile inside [e^-80, e^80]; the
// write strength beta lies in [0, 1] (section 3.1: beta scales both the erase and
// the write of the delta rule).  A NaN fails both tests.
//
// One pass per tensor: every thread counts the elements outside the domain in a
// grid-stride loop and keeps the smallest such flat index; the counts and
// indices are reduced inside the workgroup, then folded into the caller's report
// with one vector atomic add and one atomic min per workgroup (integer sums and
// minima, so the result does not depend on the order).  Two one-thread kernels
// initialise the report and turn "none found" into -1.
#include <climits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kVT = 256;
constexpr int kVBlocks = 2048;

__global__ void report_init(long long *report)
{
    report[0] = 0;
    report[1] = LLONG_MAX;
    report[2] = 0;
    report[3] = LLONG_MAX;
}

__global__ void report_finish(long long *report)
{
    if (report[1] == LLONG_MAX)
        report[1] = -1;
    if (report[3] == LLONG_MAX)
        report[3] = -1;
}

template <typename E>
__global__ __launch_bounds__(kVT) void count_outside(const E *__restrict__ x, long n, float lo, float hi,
                                                      long long *report)
{
    unsigned long long c = 0;
    long long f = LLONG_MAX;
    for (long i = (long)blockIdx.x * kVT + threadIdx.x; i < n; i += (long)gridDim.x * kVT) {
        const float v = to_f(x[i]);
        if (!(v >= lo && v <= hi)) {
            ++c;
            f = i < f ? i : f;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        c += __shfl_xor(c, off, 64);
        const long long o = __shfl_xor(f, off, 64);
        f = o < f ? o : f;
    }
    __shared__ unsigned long long sc[kVT / 64];
    __shared__ long long sf[kVT / 64];
    if ((threadIdx.x & 63) == 0) {
        sc[threadIdx.x >> 6] = c;
        sf[threadIdx.x >> 6] = f;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kVT / 64; ++w) {
            c += sc[w];
            f = sf[w] < f ? sf[w] : f;
        }
        if (c) {
            atomicAdd(reinterpret_cast<unsigned long long *>(report), c);
            atomicMin(report + 1, f);
        }
    }
}

template <typename E>
hipError_t count(const void *x, long n, float lo, float hi, long long *report, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    long blocks = (n + kVT - 1) / kVT;
    if (blocks > kVBlocks)
        blocks = kVBlocks;
    hipLaunchKernelGGL((count_outside<E>), dim3((unsigned)blocks), dim3(kVT), 0, stream, (const E *)x, n, lo, hi,
                       report);
    return hipGetLastError();
}

} // namespace

hipError_t launch_validate(const void *g, const void *beta, long long *report, long ng, long nb, bool fp32,
                           hipStream_t stream)
{
    hipLaunchKernelGGL(report_init, dim3(1), dim3(1), 0, stream, report);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    e = fp32 ? count<float>(g, ng, -5.f, 0.f, report, stream) : count<__bf16>(g, ng, -5.f, 0.f, report, stream);
    if (e != hipSuccess)
        return e;
    e = fp32 ? count<float>(beta, nb, 0.f, 1.f, report + 2, stream)
             : count<__bf16>(beta, nb, 0.f, 1.f, report + 2, stream);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(report_finish, dim3(1), dim3(1), 0, stream, report);
    return hipGetLastError();
}

namespace {

// Workgroup i of the launch records the XCD it runs on (hardware register
// XCC_ID).  The dynamic LDS the launch requests is never touched: it only makes
// each workgroup take as much of a CU as the kernels whose placement is checked.
__global__ __launch_bounds__(64) void placement_kernel(int *xcd, int n)
{
    const int i = blockIdx.x;
    if (threadIdx.x == 0 && i < n)
        xcd[i] = hw_xcd();
}

} // namespace

hipError_t launch_workgroup_xcds(int *xcd, int n, int lds_bytes, hipStream_t stream)
{
    hipError_t e = hipFuncSetAttribute((const void *)placement_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       lds_bytes);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(placement_kernel, dim3((unsigned)n), dim3(64), (unsigned)lds_bytes, stream, xcd, n);
    return hipGetLastError();
}

} // namespace kda
