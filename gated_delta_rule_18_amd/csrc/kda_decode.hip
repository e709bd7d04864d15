// kda_decode.hip -- one KDA decode step on gfx950.
//
// Method: page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section 3.2:
// the decode interface (x_t, S_{t-1}, C^conv_{t-1}) -> (y_t, S_t, C^conv_t); the
// input branches q, k = L2Norm(Swish(ShortConv(.))), v = Swish(ShortConv(.));
// and the one-token edit Sbar = Diag(alpha) S, vhat = Sbar^T k,
// S' = Sbar + beta k (v - vhat)^T, o = S'^T q (read after the write).
//
// The step is bound by HBM traffic: the 4*dk*dv-byte fp32 state of every
// (sequence, head) is read once and written once.  A workgroup owns kHP
// (sequence, head) pairs, kTPH threads each (a single head per 256-thread
// workgroup streamed the in-place read-modify-write ~8 % slower on gfx950);
// per head:
//   * each thread holds a float4 column strip of ROWS key rows of S in
//     registers from the read to the write, so HBM sees exactly one read and
//     one write of the state (loads are issued first, before the conv work);
//   * 64 consecutive lanes read rows 512 or 256 contiguous bytes wide;
//   * the readout does not re-read S': with d = v - vhat,
//       o = S'^T q = Sbar^T q + beta (q . k) d,
//     so both column sums (Sbar^T k and Sbar^T q) come out of one pass.
//
// The gated variant (kda_decode_step_gated) also applies the output exposure
// gate of the same section's output equation before W_o: the threads that hold
// o (lanes 0 .. dv/4-1 of wavefront 0, four columns each) reduce its sum of
// squares and write y = Sigmoid(gate) * o / sqrt(mean o^2 + eps) * w instead
// of o, so o never makes a round trip through HBM.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kHP = 2;                // heads per workgroup
constexpr int kTPH = 128;             // threads per head
constexpr int kThreads = kHP * kTPH;
constexpr int kWidth = 4;
constexpr float kL2Eps = 1e-6f;

__device__ __forceinline__ void load2(const __bf16 *p, float &a, float &b)
{
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    v2 x = *reinterpret_cast<const v2 *>(p);
    a = (float)x[0];
    b = (float)x[1];
}
__device__ __forceinline__ void load2(const float *p, float &a, float &b)
{
    float2 x = *reinterpret_cast<const float2 *>(p);
    a = x.x;
    b = x.y;
}
__device__ __forceinline__ void store2(__bf16 *p, float a, float b)
{
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    v2 x;
    x[0] = (__bf16)a;
    x[1] = (__bf16)b;
    *reinterpret_cast<v2 *>(p) = x;
}
__device__ __forceinline__ void store2(float *p, float a, float b)
{
    *reinterpret_cast<float2 *>(p) = make_float2(a, b);
}
__device__ __forceinline__ void store4(__bf16 *p, float a, float b, float c, float d)
{
    typedef __bf16 v4 __attribute__((ext_vector_type(4)));
    v4 x;
    x[0] = (__bf16)a;
    x[1] = (__bf16)b;
    x[2] = (__bf16)c;
    x[3] = (__bf16)d;
    *reinterpret_cast<v4 *>(p) = x;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d)
{
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

__device__ __forceinline__ float swish(float u) { return u / (1.0f + exp_f(-u)); }

template <int DK, int DV, typename E, bool GATED>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const E *__restrict__ q_pre, const E *__restrict__ k_pre, const E *__restrict__ v_pre,
    const float *__restrict__ conv_w, E *__restrict__ conv_cache, int oldest,
    const E *__restrict__ g, const E *__restrict__ beta, float *__restrict__ S,
    E *__restrict__ o, int H, long heads, const E *__restrict__ gate, const float *__restrict__ norm_w,
    float eps)
{
    constexpr int NCH = 2 * DK + DV;      // conv channels q | k | v
    constexpr int CG = DV / 4;            // float4 column groups
    constexpr int RG = kTPH / CG;         // row groups
    constexpr int ROWS = DK / RG;         // rows per thread
    constexpr int NW = kTPH / 64;         // wavefronts per head
    static_assert(kTPH % 64 == 0 && CG < 64 && ROWS >= 1 && RG * ROWS == DK, "shape");

    // head slot hs of the workgroup owns (sequence * H + head) nh; in a ragged
    // last workgroup a slot past the end redoes the last head's arithmetic (its
    // barriers are the workgroup's) and writes nothing
    const int hs = threadIdx.x / kTPH;
    const long nh_raw = (long)blockIdx.x * kHP + hs;
    const bool live = nh_raw < heads;
    const long nh = live ? nh_raw : heads - 1;
    const int h = (int)(nh % H);
    const int t = threadIdx.x % kTPH;
    const int cg = t % CG, rg = t / CG;
    const int lane = t & 63, wave = t >> 6;

    __shared__ float act_s[kHP][NCH];
    __shared__ float alpha_s[kHP][DK];
    __shared__ float red_s[kHP][NW][2 * DV];
    __shared__ float scal_s[kHP][3];
    float *act = act_s[hs], *alpha = alpha_s[hs], *scal = scal_s[hs];
    float (*red)[2 * DV] = red_s[hs];

    // 1. the state strip, loaded before anything else so the reads are in flight
    float *Sp = S + (size_t)nh * DK * DV;
    f32x4 s[ROWS];
#pragma unroll
    for (int j = 0; j < ROWS; ++j)
        s[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sp + (size_t)(rg + RG * j) * DV) + cg);

    // the gate pre-activations of this thread's four output columns (gated variant)
    float gv[4] = {0.f, 0.f, 0.f, 0.f}, wv[4] = {1.f, 1.f, 1.f, 1.f};
    if (GATED && rg == 0) {
        load2(gate + (size_t)nh * DV + 4 * cg, gv[0], gv[1]);
        load2(gate + (size_t)nh * DV + 4 * cg + 2, gv[2], gv[3]);
        if (norm_w) {
            const float4 w4 = *reinterpret_cast<const float4 *>(norm_w + 4 * cg);
            wv[0] = w4.x, wv[1] = w4.y, wv[2] = w4.z, wv[3] = w4.w;
        }
    }

    // 2. ShortConv over the window (3 cached tokens, oldest first, then x_t) + Swish
    for (int c2 = t; c2 < NCH / 2; c2 += kTPH) {
        const int c = 2 * c2;
        const E *src;
        int off;
        if (c < DK) {
            src = q_pre + (size_t)nh * DK;
            off = c;
        } else if (c < 2 * DK) {
            src = k_pre + (size_t)nh * DK;
            off = c - DK;
        } else {
            src = v_pre + (size_t)nh * DV;
            off = c - 2 * DK;
        }
        float x0, x1;
        load2(src + off, x0, x1);
        const float4 w0 = *reinterpret_cast<const float4 *>(conv_w + ((size_t)h * NCH + c) * kWidth);
        const float4 w1 = *reinterpret_cast<const float4 *>(conv_w + ((size_t)h * NCH + c + 1) * kWidth);
        E *cache = conv_cache + (size_t)nh * (kWidth - 1) * NCH;
        const float wa0[3] = {w0.x, w0.y, w0.z}, wa1[3] = {w1.x, w1.y, w1.z};
        float u0 = w0.w * x0, u1 = w1.w * x1;
#pragma unroll
        for (int j = 0; j < kWidth - 1; ++j) {
            int slot = oldest + j;
            slot = slot >= kWidth - 1 ? slot - (kWidth - 1) : slot;
            float a0, a1;
            load2(cache + slot * NCH + c, a0, a1);
            u0 += wa0[j] * a0;
            u1 += wa1[j] * a1;
        }
        if (live)
            store2(cache + oldest * NCH + c, x0, x1);   // x_t replaces the oldest token
        act[c] = swish(u0);
        act[c + 1] = swish(u1);
    }
    for (int i = t; i < DK; i += kTPH)
        alpha[i] = exp_f(to_f(g[(size_t)nh * DK + i]));
    __syncthreads();

    // 3. L2Norm scales of q and k, and q . k, by wavefront 0
    if (wave == 0) {
        float sq = 0.f, sk = 0.f, qk = 0.f;
        for (int c = lane; c < DK; c += 64) {
            const float a = act[c], b = act[DK + c];
            sq += a * a;
            sk += b * b;
            qk += a * b;
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        qk = wave_sum(qk);
        if (lane == 0) {
            const float rq = rsqrtf(sq + kL2Eps), rk = rsqrtf(sk + kL2Eps);
            scal[0] = rq;
            scal[1] = rk;
            scal[2] = qk * rq * rk;
        }
    }
    __syncthreads();
    const float rq = scal[0], rk = scal[1], qdotk = scal[2];
    const float bt = to_f(beta[nh]);

    // 4. decay the rows, then the two column sums over this thread's rows
    float vh[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < ROWS; ++j) {
        const int i = rg + RG * j;
        const float a = alpha[i], kk = act[DK + i] * rk, qq = act[i] * rq;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s[j][c] *= a;
            vh[c] += s[j][c] * kk;
            pq[c] += s[j][c] * qq;
        }
    }
    // row groups inside a wavefront are CG lanes apart
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            vh[c] += __shfl_xor(vh[c], off, 64);
            pq[c] += __shfl_xor(pq[c], off, 64);
        }
    }
    if (lane < CG) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            red[wave][4 * cg + c] = vh[c];
            red[wave][DV + 4 * cg + c] = pq[c];
        }
    }
    __syncthreads();

    // 5. the edit S' = Sbar + beta k d^T and the readout o = Sbar^T q + beta (q.k) d
    float d[4], p[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float vs = 0.f, ps = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            vs += red[w][4 * cg + c];
            ps += red[w][DV + 4 * cg + c];
        }
        d[c] = act[2 * DK + 4 * cg + c] - vs;
        p[c] = ps;
    }
#pragma unroll
    for (int j = 0; j < ROWS; ++j) {
        const int i = rg + RG * j;
        const float bk = bt * act[DK + i] * rk;
        f32x4 r = s[j];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            r[c] += bk * d[c];
        if (live)
            __builtin_nontemporal_store(r, reinterpret_cast<f32x4 *>(Sp + (size_t)i * DV) + cg);
    }
    const float bq = bt * qdotk;
    float ov[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        ov[c] = p[c] + bq * d[c];
    if constexpr (GATED) {
        // lanes 0 .. CG-1 of wavefront 0 hold the head's row of o; xor offsets
        // below CG keep the reduction inside them
        if (wave == 0) {
            float ss = rg == 0 ? ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3] : 0.f;
#pragma unroll
            for (int off = CG / 2; off > 0; off >>= 1)
                ss += __shfl_xor(ss, off, 64);
            if (rg == 0) {
                const float r = rsqrtf(ss * (1.0f / DV) + eps);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    ov[c] = __builtin_amdgcn_rcpf(1.0f + exp_f(-gv[c])) * ov[c] * r * wv[c];
            }
        }
    }
    if (rg == 0 && live)
        store4(o + (size_t)nh * DV + 4 * cg, ov[0], ov[1], ov[2], ov[3]);
}

template <int DK, int DV, typename E>
hipError_t launch(const void *q_pre, const void *k_pre, const void *v_pre, const float *conv_w,
                  void *conv_cache, int oldest, const void *g, const void *beta, float *S, void *o,
                  int N, int H, const OutputGate &og, hipStream_t stream)
{
    const long heads = (long)N * H;
    if (heads == 0)
        return hipSuccess;
    const long blocks = (heads + kHP - 1) / kHP;
    if (og.gate)
        hipLaunchKernelGGL((decode_kernel<DK, DV, E, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, (const E *)q_pre, (const E *)k_pre, (const E *)v_pre, conv_w,
                           (E *)conv_cache, oldest, (const E *)g, (const E *)beta, S, (E *)o, H, heads,
                           (const E *)og.gate, og.w, og.eps);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, E, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, (const E *)q_pre, (const E *)k_pre, (const E *)v_pre, conv_w,
                           (E *)conv_cache, oldest, (const E *)g, (const E *)beta, S, (E *)o, H, heads,
                           (const E *)nullptr, (const float *)nullptr, 0.f);
    return hipGetLastError();
}

template <typename E>
hipError_t dispatch(int dk, int dv, const void *q_pre, const void *k_pre, const void *v_pre,
                    const float *conv_w, void *conv_cache, int oldest, const void *g,
                    const void *beta, float *S, void *o, int N, int H, const OutputGate &og,
                    hipStream_t stream)
{
#define KDA_DECODE_CASE(A, B)                                                                    \
    if (dk == A && dv == B)                                                                     \
        return launch<A, B, E>(q_pre, k_pre, v_pre, conv_w, conv_cache, oldest, g, beta, S, o, N, \
                               H, og, stream);
    KDA_DECODE_CASE(128, 128)
    KDA_DECODE_CASE(128, 64)
    KDA_DECODE_CASE(64, 128)
    KDA_DECODE_CASE(64, 64)
#undef KDA_DECODE_CASE
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_decode_step(const void *q_pre, const void *k_pre, const void *v_pre,
                              const float *conv_w, void *conv_cache, int oldest_slot,
                              const void *g, const void *beta, float *S, void *o, int N, int H,
                              int dk, int dv, bool fp32, const OutputGate &og, hipStream_t stream)
{
    if (fp32)
        return dispatch<float>(dk, dv, q_pre, k_pre, v_pre, conv_w, conv_cache, oldest_slot, g,
                               beta, S, o, N, H, og, stream);
    return dispatch<__bf16>(dk, dv, q_pre, k_pre, v_pre, conv_w, conv_cache, oldest_slot, g, beta,
                            S, o, N, H, og, stream);
}

} // namespace kda
