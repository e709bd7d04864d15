// kda_gate.hip -- the output exposure gate of a KDA layer on gfx950
// (kda_output_gate).
//
// Method: page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section 3.2,
// output equation y_t = W_o[Sigmoid(W_g x_t) (.) RMSNorm(o~_t)].  This kernel
// computes the bracket; W_o (and W_g x_t, passed in as `gate`) are the
// caller's GEMMs.  The section says RMSNorm steadies each head's readout, so
// the norm runs over the dv channels of one (row, head), with a per-channel
// weight w shared by the heads:
//     y[r,h,c] = Sigmoid(gate[r,h,c]) * o[r,h,c] / sqrt(mean_c' o[r,h,c']^2 + eps) * w[c]
//
// The kernel is bound by HBM traffic (read o and gate, write y: 3 dv elements
// per unit).  LPU = dv / 8 consecutive lanes own one unit, 8 contiguous
// elements each (one 16-byte load per tensor in bf16, two in fp32); the sum of
// squares is reduced over the unit's lanes with xor shuffles, which stay
// inside the unit's aligned group of LPU lanes.  Wavefronts stride over the
// units with kGateUnroll units in flight per lane.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kGateThreads = 256;
// two resident workgroups per CU, each lane with 16 units' loads in flight: on
// gfx950 this streamed 27 % faster than 8 workgroups per CU with 2 units each
constexpr int kGateBlocksPerCU = 2;
constexpr int kGateUnroll = 16;
constexpr int kCUs = 256;

template <typename E> struct Oct;
template <> struct Oct<__bf16> {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    u4 r;
    static __device__ __forceinline__ Oct load(const __bf16 *p)
    {
        return Oct{__builtin_nontemporal_load(reinterpret_cast<const u4 *>(p))};
    }
    __device__ __forceinline__ float get(int i) const
    {
        const unsigned x = r[i >> 1];
        return __uint_as_float((i & 1) ? (x & 0xffff0000u) : (x << 16));
    }
    static __device__ __forceinline__ void store(__bf16 *p, const float *v)
    {
        u4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            typedef __bf16 v2 __attribute__((ext_vector_type(2)));
            v2 t;
            t[0] = (__bf16)v[2 * i];
            t[1] = (__bf16)v[2 * i + 1];
            x[i] = __builtin_bit_cast(unsigned, t);
        }
        __builtin_nontemporal_store(x, reinterpret_cast<u4 *>(p));
    }
};
template <> struct Oct<float> {
    f32x4 a, b;
    static __device__ __forceinline__ Oct load(const float *p)
    {
        return Oct{__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p)),
                   __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + 1)};
    }
    __device__ __forceinline__ float get(int i) const { return i < 4 ? a[i] : b[i - 4]; }
    static __device__ __forceinline__ void store(float *p, const float *v)
    {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4 *>(p) + 1);
    }
};

template <typename E, int DV>
__device__ __forceinline__ void gate_unit(const Oct<E> &xo, const Oct<E> &xg, const float *wv, float eps,
                                          E *dst)
{
    constexpr int LPU = DV / 8;
    float x[8], ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[i] = xo.get(i);
        ss += x[i] * x[i];
    }
#pragma unroll
    for (int off = LPU / 2; off > 0; off >>= 1)
        ss += __shfl_xor(ss, off, 64);
    const float r = gate_rms(ss, 1.0f / DV, eps);
    float yv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        yv[i] = gate_elem(x[i], xg.get(i), r, wv[i]);
    Oct<E>::store(dst, yv);
}

template <typename E, int DV>
__global__ __launch_bounds__(kGateThreads) void gate_kernel(const E *__restrict__ o, const E *__restrict__ gate,
                                                            const float *__restrict__ w, E *y, long units,
                                                            float eps)
{
    constexpr int LPU = DV / 8;           // lanes per unit
    constexpr int UPW = 64 / LPU;         // units per wavefront
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPU, slot = lane / LPU;
    float wv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        wv[i] = w ? w[8 * sub + i] : 1.f;
    const long wave = (long)blockIdx.x * (kGateThreads / 64) + (threadIdx.x >> 6);
    const long stride = (long)gridDim.x * (kGateThreads / 64) * UPW;
    long u = wave * UPW + slot;
    // kGateUnroll units per lane per iteration: all their loads are issued first
    for (; u + (kGateUnroll - 1) * stride < units; u += kGateUnroll * stride) {
        Oct<E> xo[kGateUnroll], xg[kGateUnroll];
#pragma unroll
        for (int j = 0; j < kGateUnroll; ++j) {
            const long e = (u + j * stride) * DV + 8 * sub;
            xo[j] = Oct<E>::load(o + e);
            xg[j] = Oct<E>::load(gate + e);
        }
#pragma unroll
        for (int j = 0; j < kGateUnroll; ++j)
            gate_unit<E, DV>(xo[j], xg[j], wv, eps, y + (u + j * stride) * DV + 8 * sub);
    }
    for (; u < units; u += stride) {
        const long e0 = u * DV + 8 * sub;
        gate_unit<E, DV>(Oct<E>::load(o + e0), Oct<E>::load(gate + e0), wv, eps, y + e0);
    }
}

template <typename E, int DV>
hipError_t launch(const void *o, const void *gate, const float *w, void *y, long units, float eps,
                  hipStream_t stream)
{
    constexpr long per_block = (kGateThreads / 64) * (64 / (DV / 8));
    long blocks = (units + per_block - 1) / per_block;
    if (blocks > (long)kCUs * kGateBlocksPerCU)
        blocks = (long)kCUs * kGateBlocksPerCU;
    hipLaunchKernelGGL((gate_kernel<E, DV>), dim3((unsigned)blocks), dim3(kGateThreads), 0, stream,
                       (const E *)o, (const E *)gate, w, (E *)y, units, eps);
    return hipGetLastError();
}

} // namespace

hipError_t launch_output_gate(const void *o, const void *gate, const float *w, void *y, long units,
                              int dv, float eps, bool fp32, hipStream_t stream)
{
    if (units == 0)
        return hipSuccess;
    if (fp32)
        return dv == 128 ? launch<float, 128>(o, gate, w, y, units, eps, stream)
                         : launch<float, 64>(o, gate, w, y, units, eps, stream);
    return dv == 128 ? launch<__bf16, 128>(o, gate, w, y, units, eps, stream)
                     : launch<__bf16, 64>(o, gate, w, y, units, eps, stream);
}

} // namespace kda
