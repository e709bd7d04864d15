// kda_device.h -- device-side helpers shared by the KDA kernels (gfx950 only).
//
// Element types: __bf16 (bf16 mode) or float (fp32 test mode).  Conversions to
// and from float use the compiler's native __bf16 casts, which gfx950 lowers to
// its round-to-nearest-even conversion instruction.
#pragma once
#include <hip/hip_runtime.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename E> struct Vec;
template <> struct Vec<__bf16> {
    typedef __bf16 v4 __attribute__((ext_vector_type(4)));
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
};
template <> struct Vec<float> {
    typedef float v4 __attribute__((ext_vector_type(4)));
    typedef float v8 __attribute__((ext_vector_type(8)));
};

__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename E> __device__ __forceinline__ E from_f(float x) { return (E)x; }

template <typename E>
__device__ __forceinline__ typename Vec<E>::v4 cvt4(f32x4 x)
{
    typename Vec<E>::v4 r;
    r[0] = (E)x[0];
    r[1] = (E)x[1];
    r[2] = (E)x[2];
    r[3] = (E)x[3];
    return r;
}

template <typename V4>
__device__ __forceinline__ auto cat8(V4 a, V4 b)
{
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// D += A * B over a 32-deep contraction slice, 16x16 output tile.
// Lane l supplies row (l % 16) of A and column (l % 16) of B; its 8 operand
// elements are 8 contraction indices.  Which 8 indices a lane holds is up to
// the caller, as long as A and B agree element by element: the hardware pairs
// element e of A's lane (i + 16 g) with element e of B's lane (n + 16 g).
__device__ __forceinline__ f32x4 mma32(Vec<__bf16>::v8 a, Vec<__bf16>::v8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(Vec<float>::v8 a, Vec<float>::v8 b, f32x4 c)
{
#pragma unroll
    for (int e = 0; e < 8; ++e)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}
// Same with a 16-deep slice (4 elements per lane).  The bf16 form zero-pads to
// the 32-deep instruction instead of using the 16-deep one: a kernel then uses a
// single MFMA opcode, so an accumulation never chains two MFMAs of different
// pass counts onto the same accumulator (this toolchain was seen to issue such
// a pair back to back without the wait states the dependency needs).
__device__ __forceinline__ f32x4 mma16(Vec<__bf16>::v4 a, Vec<__bf16>::v4 b, f32x4 c)
{
    const Vec<__bf16>::v4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat8(a, z), cat8(b, z), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(Vec<float>::v4 a, Vec<float>::v4 b, f32x4 c)
{
#pragma unroll
    for (int e = 0; e < 4; ++e)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

// e^x through the hardware base-2 exponential.  The rounding of x * log2(e)
// costs a relative error of about |x| * 2^-24 (5e-6 at x = -80).
__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// e^x to a few ulp over the whole range the kernels use (|x| <= 80): the product
// y = x * log2(e) is rounded, its rounding error is recovered exactly with an FMA
// (the error-free product transformation) and added with the tail of log2(e) as
// a first-order correction, 2^(y + d) = 2^y (1 + d ln 2), |d| < 2^-17.
__device__ __forceinline__ float exp_acc(float x)
{
    const float L = 1.44269502162933349609375f;     // log2(e) rounded to fp32
    const float Lt = 1.9259629911e-8f;               // log2(e) - L
    const float y = x * L;
    const float d = __builtin_fmaf(x, L, -y) + x * Lt;
    return __builtin_amdgcn_exp2f(y) * __builtin_fmaf(d, 0.69314718055994531f, 1.f);
}

// 1 / x from the hardware reciprocal refined by one Newton step.
__device__ __forceinline__ float rcp_acc(float x)
{
    const float r = __builtin_amdgcn_rcpf(x);
    return __builtin_fmaf(__builtin_fmaf(-x, r, 1.f), r, r);
}

// The output exposure gate (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读",
// section 3.2, output equation), as every kernel that applies it evaluates it:
// r = 1 / sqrt(ss / n + eps) for a (row, head) whose n readout values have the
// sum of squares ss, then y = Sigmoid(gate) * o * r * w per element.
__device__ __forceinline__ float gate_rms(float ss, float inv_n, float eps) { return rsqrtf(ss * inv_n + eps); }
__device__ __forceinline__ float gate_elem(float o, float gt, float r, float w)
{
    return __builtin_amdgcn_rcpf(1.0f + exp_f(-gt)) * o * r * w;
}

// The XCD (accelerator complex die) the calling wavefront runs on: hardware
// register 20 (XCC_ID), bits [3:0].  A launch's workgroups go round-robin over
// the 8 XCDs of this part, so workgroups i and i + 8 share one XCD and its L2,
// which the hand-offs between workgroups rely on (which XCD takes workgroup 0
// varies from launch to launch).  Hand-off words carry their writer's XCD in bits
// [30:28] so that the reader checks the assumption (and marks its results NaN)
// instead of reading another L2's stale data.
__device__ __forceinline__ int hw_xcd() { return (int)__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20); }
constexpr int kXcdShift = 28;
constexpr int kCountMask = (1 << kXcdShift) - 1;
__device__ __forceinline__ int tag_xcd(int count, int xcd) { return count | (xcd << kXcdShift); }
__device__ __forceinline__ int word_count(int w) { return w & kCountMask; }
__device__ __forceinline__ int word_xcd(int w) { return (int)((unsigned)w >> kXcdShift); }

// Sum over the 64 lanes of a wavefront (result valid in every lane).
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

} // namespace kda
