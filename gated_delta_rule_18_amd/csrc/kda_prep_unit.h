// kda_prep_unit.h -- the prefill preprocessing of one unit of work, shared by
// the preprocessing kernel (kda_prefill_prep) and the prep workers of the fused
// prefill (kda_chunk_fwd_from_proj).  Device code only.
//
// Method: page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读"
//   section 3.2, input branches: q, k = L2Norm(Swish(ShortConv(W x))),
//                v = Swish(ShortConv(W_v x)), beta = Sigmoid(W_beta x);
//   section 3.3, lower-bounded decay: g = g_min * Sigmoid(e^{A^h} z), g_min = -5,
//                one scalar A^h per head.
// ShortConv is depthwise and causal, width 4, tap 0 on the oldest token, with
// the window reaching back into a caller-given history of the 3 tokens before
// the first one (the decode conv cache, oldest first).
//
// A unit is two heads (flat (sequence, head) indices bhA and bhB) over one
// kTT-token tile, worked by four wavefronts; every wavefront runs one kind of
// work on all of its lanes (no divergent roles inside a wavefront), 4 channels
// per lane:
//   wavefronts 0, 1: q (first dk/4 lanes) and k (next dk/4 lanes) of head bhA
//                    (bhB): conv, Swish, then the L2 norm as a reduction over
//                    the dk/4 lanes of the group;
//   wavefront 2:     v of bhA (lanes 0..) and of bhB (lanes 32..): conv, Swish;
//   wavefront 3:     the gate input z of bhA (lanes 0..) and bhB (lanes 32..);
//   wavefronts 2, 3 also map beta of the tile's tokens (lane = token mod 64) for
//                    bhA and bhB respectively.
// A conv lane walks the tile token by token keeping its last three inputs in
// registers; loads run KU tokens ahead.  A token's result does not depend on
// KU or on where the token falls in the walk.
#pragma once
#include "kda_device.h"

namespace kda {
namespace {


constexpr int kTT = 128;                 // tokens per tile
constexpr int kW = 4;                    // conv width
constexpr float kL2Eps = 1e-6f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kGMin = -5.0f;

__device__ __forceinline__ f32x4 ld4(const __bf16 *p)
{
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
    return f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                 __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

__device__ __forceinline__ void st4(__bf16 *p, f32x4 x)
{
    *reinterpret_cast<typename Vec<__bf16>::v4 *>(p) = cvt4<__bf16>(x);
}
__device__ __forceinline__ void st4(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }

// 1 / (1 + e^{-u}) with the hardware exponential and reciprocal; saturates to
// 0 and 1 (e^{-u} = inf gives 0).
__device__ __forceinline__ float sigmoid_f(float u)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * u));
}

// Sum over the `n` lanes of an aligned lane group (n a power of two <= 32).
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
#pragma unroll
    for (int off = N / 2; off > 0; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

// What a wavefront's lanes compute.
enum Role { kQK = 0, kV = 1, kGate = 2 };

// The token walk of one lane over its tile: 4 channels starting at element c4
// of a row of D elements of `src`, rows t0 .. t0 + n - 1 of unit (b, h) at
// `base` (element offset of row t0), `step` elements between token rows.
// kQK / kV lanes: conv over (hist, x_t) with taps w, Swish, and for kQK the L2
// norm over the lane group of NG lanes; kGate lanes: g = -5 Sigmoid(eA z).
template <int R, int NG, int KU, typename E>
__device__ __forceinline__ void walk(const E *src, E *dst, long base, long step, int n, const f32x4 *w,
                                     f32x4 *hist, float eA, bool active)
{
    for (int tb = 0; tb < n; tb += KU) {
        // loads first (rows past the tile are clamped to its last token and not used)
        f32x4 xin[KU];
#pragma unroll
        for (int i = 0; i < KU; ++i)
            xin[i] = ld4(src + base + (tb + i < n ? tb + i : n - 1) * step);
#pragma unroll
        for (int i = 0; i < KU; ++i) {
            if (tb + i >= n)
                break;
            f32x4 y;
            if constexpr (R == kGate) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y[e] = kGMin * sigmoid_f(eA * xin[i][e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // explicit fused multiply-adds in a fixed order: a token's result
                    // must not depend on where it falls in the unrolled walk
                    const float u = __builtin_fmaf(w[3][e], xin[i][e],
                                    __builtin_fmaf(w[2][e], hist[2][e],
                                    __builtin_fmaf(w[1][e], hist[1][e], w[0][e] * hist[0][e])));
                    y[e] = u * sigmoid_f(u);
                }
                hist[0] = hist[1];
                hist[1] = hist[2];
                hist[2] = xin[i];
                if constexpr (R == kQK) {
                    const float ss = group_sum<NG>(__builtin_fmaf(y[3], y[3], __builtin_fmaf(y[2], y[2],
                                                   __builtin_fmaf(y[1], y[1], y[0] * y[0]))));
                    y *= __builtin_amdgcn_rsqf(ss + kL2Eps);
                }
            }
            if (active)
                st4(dst + base + (tb + i) * step, y);
        }
    }
}


// One unit: heads bhA and bhB (bhB < 0: none) over tile `tile`; `wave` (0..3) is
// the wavefront's role in the unit.  Idle lanes read valid memory and store
// nothing.  The tile-0 unit also writes conv_final (when not null): the last 3
// pre-activations of the sequence, read before any of them is written
// (conv_final may be conv_init itself).
template <typename E, int DK, int DV, int KU>
__device__ __forceinline__ void prep_unit(const E *__restrict__ q_pre, const E *__restrict__ k_pre,
                                          const E *__restrict__ v_pre, const float *__restrict__ conv_w,
                                          const E *conv_init, const E *__restrict__ z, const float *__restrict__ A,
                                          const E *__restrict__ beta_logit, E *q, E *k, E *v, E *g, E *beta,
                                          E *conv_final, int T, int H, int bhA, int bhB, int tile, int wave,
                                          int lane)
{
    constexpr int NCH = 2 * DK + DV;
    constexpr int QK = DK / 4, VQ = DV / 4;     // 4-channel lanes per tensor
    static_assert(2 * QK <= 64 && VQ <= 32 && QK <= 32, "lane budget");
    const int t0 = tile * kTT;
    const int n = T - t0 < kTT ? T - t0 : kTT;           // tokens in this tile

    // this lane's (sequence, head), tensor and first channel
    int bh, c4, cc;                                     // cc = conv channel (order q | k | v)
    const E *src;
    E *dst;
    bool active;
    if (wave < 2) {
        bh = wave == 0 ? bhA : bhB;
        const bool isk = lane >= QK;
        c4 = 4 * (isk ? lane - QK : lane);
        cc = isk ? DK + c4 : c4;
        src = isk ? k_pre : q_pre;
        dst = isk ? k : q;
        active = lane < 2 * QK;
    } else {
        bh = (lane >> 5) ? bhB : bhA;
        c4 = 4 * (lane & 31);
        cc = 2 * DK + c4;
        src = wave == 2 ? v_pre : z;
        dst = wave == 2 ? v : g;
        active = c4 < (wave == 2 ? DV : DK);
    }
    active = active && bh >= 0;
    if (!active)
        bh = bhA, c4 = 0, cc = 0;
    const int b = bh / H, h = bh % H;
    const long tokb = (long)b * T;
    const int D = wave == 2 ? DV : DK;
    const long step = (long)H * D;
    const long base = ((tokb + t0) * H + h) * (long)D + c4;

    // ---- beta = Sigmoid(logit): wavefront 2 for bhA, 3 for bhB, lane = token ------
    if (wave >= 2) {
        const int hb = wave == 2 ? bhA : bhB;
        if (hb >= 0) {
            const long tb = (long)(hb / H) * T;
            const int hh = hb % H;
            for (int tt = lane; tt < n; tt += 64) {
                const long r = (tb + t0 + tt) * H + hh;
                beta[r] = (E)sigmoid_f(to_f(beta_logit[r]));
            }
        }
    }

    if (wave == 3) {
        walk<kGate, 32, KU>(src, dst, base, step, n, nullptr, nullptr, expf(A[h]), active);
        return;
    }

    // ---- conv lanes (q, k, v): taps, history, then the token walk --------------
    f32x4 w[kW];                                // w[j][e] = tap j of channel cc + e
    f32x4 hist[kW - 1];                         // inputs of tokens t-3, t-2, t-1
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const f32x4 we = *reinterpret_cast<const f32x4 *>(conv_w + ((long)h * NCH + cc + e) * kW);
#pragma unroll
        for (int j = 0; j < kW; ++j)
            w[j][e] = we[j];
    }
    const E *ci = conv_init ? conv_init + (long)bh * (kW - 1) * NCH + cc : nullptr;
#pragma unroll
    for (int j = 0; j < kW - 1; ++j) {
        const int t = t0 - (kW - 1) + j;
        if (t >= 0)
            hist[j] = ld4(src + base + (long)(t - t0) * step);
        else if (ci)
            hist[j] = ld4(ci + ((kW - 1) + t) * NCH);
        else
            hist[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4 fin[kW - 1];
    const bool write_final = tile == 0 && conv_final;
    if (write_final) {
#pragma unroll
        for (int j = 0; j < kW - 1; ++j) {
            const int t = T - (kW - 1) + j;
            if (t >= 0)
                fin[j] = ld4(src + base + (long)(t - t0) * step);
            else if (ci)
                fin[j] = ld4(ci + ((kW - 1) + t) * NCH);
            else
                fin[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    if (wave < 2)
        walk<kQK, QK, KU>(src, dst, base, step, n, w, hist, 0.f, active);
    else
        walk<kV, 32, KU>(src, dst, base, step, n, w, hist, 0.f, active);

    if (write_final && active) {
#pragma unroll
        for (int j = 0; j < kW - 1; ++j)
            st4(conv_final + ((long)bh * (kW - 1) + j) * NCH + cc, fin[j]);
    }
}

} // namespace
} // namespace kda
