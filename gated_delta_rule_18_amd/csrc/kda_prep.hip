// kda_prep.hip -- prefill preprocessing on gfx950 (kda_prefill_prep).
//
// Method: page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读"
//   section 3.2, input branches: q, k = L2Norm(Swish(ShortConv(W x))),
//                v = Swish(ShortConv(W_v x)), beta = Sigmoid(W_beta x);
//   section 3.3, lower-bounded decay: g = g_min * Sigmoid(e^{A^h} z), g_min = -5,
//                one scalar A^h per head.
// The projections W x are the caller's; this kernel maps their outputs (the
// pre-activations) to the q, k, v, g, beta that kda_chunk_fwd consumes.
// ShortConv is depthwise and causal, width 4, tap 0 on the oldest token, with
// the window reaching back into a caller-given history of the 3 tokens before
// the first one (the decode conv cache, oldest first).
//
// The pass is elementwise along the sequence except for the conv window and
// the two L2 norms, so it is bound by HBM traffic: every pre-activation is read
// once (plus a 3-token halo per tile, served by L2) and every output written
// once.  A workgroup of two wavefronts owns one (sequence, head, 64-token tile):
//   wavefront 0: lanes hold 4 channels each of q (first dk/4 lanes) and k (next
//                dk/4 lanes); the L2 norm is a reduction over the dk/4 lanes of
//                the group.  It also maps beta for the tile's 64 tokens (lane =
//                token).
//   wavefront 1: lanes hold 4 channels each of v (first dv/4 lanes) and of the
//                gate input z (next dk/4 lanes).
// A conv lane walks the tile token by token keeping its last three inputs in
// registers; loads run 8 tokens ahead.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kTT = 64;                  // tokens per tile
constexpr int kW = 4;                    // conv width
constexpr int kU = 8;                    // tokens loaded ahead
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

template <typename E, int DK, int DV>
__global__ __launch_bounds__(128) void prep_kernel(
    const E *__restrict__ q_pre, const E *__restrict__ k_pre, const E *__restrict__ v_pre,
    const float *__restrict__ conv_w, const E *conv_init, const E *__restrict__ z,
    const float *__restrict__ A, const E *__restrict__ beta_logit, E *__restrict__ q,
    E *__restrict__ k, E *__restrict__ v, E *__restrict__ g, E *__restrict__ beta, E *conv_final,
    int T, int H)
{
    constexpr int NCH = 2 * DK + DV;
    constexpr int QK = DK / 4, VQ = DV / 4;     // 4-channel lanes per tensor
    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t0 = tile * kTT;
    const int t1 = T - t0 < kTT ? T - t0 : kTT;          // tokens in this tile (may be <= 0 only if T == 0)
    const long tokb = (long)b * T;
    const long bh = (long)b * H + h;

    // ---- beta = Sigmoid(logit), lane = token ----------------------------------
    if (wave == 0 && lane < t1) {
        const long r = (tokb + t0 + lane) * H + h;
        beta[r] = (E)sigmoid_f(to_f(beta_logit[r]));
    }

    // this lane's role: conv tensor (0 = q, 1 = k, 2 = v), gate (3) or idle (-1)
    int role = -1, c4 = 0;                      // c4 = first channel within its tensor
    if (wave == 0) {
        if (lane < QK)
            role = 0, c4 = 4 * lane;
        else if (lane < 2 * QK)
            role = 1, c4 = 4 * (lane - QK);
    } else {
        if (lane < VQ)
            role = 2, c4 = 4 * lane;
        else if (lane < VQ + QK)
            role = 3, c4 = 4 * (lane - VQ);
    }
    const int D = role == 2 ? DV : DK;
    const E *src = role == 0 ? q_pre : role == 1 ? k_pre : role == 2 ? v_pre : z;
    E *dst = role == 0 ? q : role == 1 ? k : role == 2 ? v : g;
    const int cc = role == 0 ? c4 : role == 1 ? DK + c4 : 2 * DK + c4;   // conv channel
    if (role < 0)
        src = q_pre, dst = nullptr;
    auto row = [&](int t) { return ((tokb + t) * H + h) * (long)D + c4; };

    if (role == 3) {
        // ---- gate: g = -5 Sigmoid(e^A z) ---------------------------------------
        const float eA = expf(A[h]);
        for (int tb = 0; tb < t1; tb += kU) {
            f32x4 xin[kU];
#pragma unroll
            for (int i = 0; i < kU; ++i)
                xin[i] = ld4(src + row(t0 + (tb + i < t1 ? tb + i : t1 - 1)));
#pragma unroll
            for (int i = 0; i < kU; ++i) {
                if (tb + i >= t1)
                    break;
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y[e] = kGMin * sigmoid_f(eA * xin[i][e]);
                st4(dst + row(t0 + tb + i), y);
            }
        }
        return;
    }

    // ---- conv lanes (q, k, v): taps, history, then the token walk --------------
    f32x4 w[kW];                                // w[j][e] = tap j of channel cc + e
    f32x4 hist[kW - 1];                         // inputs of tokens t-3, t-2, t-1
    if (role >= 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x4 we = *reinterpret_cast<const f32x4 *>(conv_w + ((long)h * NCH + cc + e) * kW);
#pragma unroll
            for (int j = 0; j < kW; ++j)
                w[j][e] = we[j];
        }
#pragma unroll
        for (int j = 0; j < kW - 1; ++j) {
            const int t = t0 - (kW - 1) + j;
            if (t >= 0)
                hist[j] = ld4(src + row(t));
            else if (conv_init)
                hist[j] = ld4(conv_init + (bh * (kW - 1) + (kW - 1) + t) * NCH + cc);
            else
                hist[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // the history the next call continues from (tile 0 only): the last 3
    // pre-activations, read before any of them is written (conv_final may be
    // conv_init itself)
    f32x4 fin[kW - 1];
    const bool write_final = tile == 0 && conv_final && role >= 0;
    if (write_final) {
#pragma unroll
        for (int j = 0; j < kW - 1; ++j) {
            const int t = T - (kW - 1) + j;
            if (t >= 0)
                fin[j] = ld4(src + row(t));
            else if (conv_init)
                fin[j] = ld4(conv_init + (bh * (kW - 1) + (kW - 1) + t) * NCH + cc);
            else
                fin[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    for (int tb = 0; tb < t1; tb += kU) {
        // loads first (rows past the tile are clamped to its last token and not used)
        f32x4 xin[kU];
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const int t = t0 + (tb + i < t1 ? tb + i : t1 - 1);
            xin[i] = ld4(src + row(t));
        }
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            if (tb + i >= t1)
                break;
            f32x4 a;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float u = w[0][e] * hist[0][e] + w[1][e] * hist[1][e] + w[2][e] * hist[2][e] +
                                w[3][e] * xin[i][e];
                a[e] = u * sigmoid_f(u);
            }
            hist[0] = hist[1];
            hist[1] = hist[2];
            hist[2] = xin[i];
            // L2Norm over the group's lanes (v lanes take the same uniform path
            // and ignore the scale)
            float ss = a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3];
            ss = group_sum<QK>(ss);
            const float r = role == 2 ? 1.0f : __builtin_amdgcn_rsqf(ss + kL2Eps);
            if (role >= 0)
                st4(dst + row(t0 + tb + i), a * r);
        }
    }

    if (write_final) {
#pragma unroll
        for (int j = 0; j < kW - 1; ++j)
            st4(conv_final + (bh * (kW - 1) + j) * NCH + cc, fin[j]);
    }
}

template <typename E, int DK, int DV>
hipError_t launch(const void *q_pre, const void *k_pre, const void *v_pre, const float *conv_w,
                  const void *conv_init, const void *z, const float *A, const void *beta_logit,
                  void *q, void *k, void *v, void *g, void *beta, void *conv_final, int B, int T,
                  int H, hipStream_t stream)
{
    if ((long)B * H == 0)
        return hipSuccess;
    const int tiles = T > 0 ? (T + kTT - 1) / kTT : 1;
    hipLaunchKernelGGL((prep_kernel<E, DK, DV>), dim3(tiles, H, B), dim3(128), 0, stream,
                       (const E *)q_pre, (const E *)k_pre, (const E *)v_pre, conv_w,
                       (const E *)conv_init, (const E *)z, A, (const E *)beta_logit, (E *)q, (E *)k,
                       (E *)v, (E *)g, (E *)beta, (E *)conv_final, T, H);
    return hipGetLastError();
}

template <typename E>
hipError_t dispatch(int dk, int dv, const void *q_pre, const void *k_pre, const void *v_pre,
                    const float *conv_w, const void *conv_init, const void *z, const float *A,
                    const void *beta_logit, void *q, void *k, void *v, void *g, void *beta,
                    void *conv_final, int B, int T, int H, hipStream_t stream)
{
#define KDA_PREP_CASE(X, Y)                                                                        \
    if (dk == X && dv == Y)                                                                       \
        return launch<E, X, Y>(q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit, q, k, v, g, \
                               beta, conv_final, B, T, H, stream);
    KDA_PREP_CASE(128, 128)
    KDA_PREP_CASE(128, 64)
    KDA_PREP_CASE(64, 128)
    KDA_PREP_CASE(64, 64)
#undef KDA_PREP_CASE
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_prefill_prep(const void *q_pre, const void *k_pre, const void *v_pre,
                               const float *conv_w, const void *conv_init, const void *z,
                               const float *A, const void *beta_logit, void *q, void *k, void *v,
                               void *g, void *beta, void *conv_final, int B, int T, int H, int dk,
                               int dv, bool fp32, hipStream_t stream)
{
    if (fp32)
        return dispatch<float>(dk, dv, q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit, q,
                               k, v, g, beta, conv_final, B, T, H, stream);
    return dispatch<__bf16>(dk, dv, q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit, q, k,
                            v, g, beta, conv_final, B, T, H, stream);
}

} // namespace kda
