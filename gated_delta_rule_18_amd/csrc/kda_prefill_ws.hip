// kda_prefill_ws.hip -- warp-specialised chunkwise KDA prefill on gfx950
// (kda_chunk_fwd with chunk = 16).
//
// Method: page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读"
//   section 3.1, KDA recurrence: S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
//                                o_t = S_t^T q_t, a_t = exp(g_t) per key channel;
//   section 3.3, chunk interface (X_[c], S_in) -> (Y_[c], S_out) with
//                S_in(c+1) = S_out(c), WY/UT organisation inside a chunk;
//   section 3.3, lower-bounded decay: g >= -5, so a 16-position tile's summed
//                log-decay stays in (-80, 0] and its inverse e^{+80} fits bf16.
//
// Chunk algebra for a 16-token chunk with incoming state S and chunk-relative
// G_r = sum_{s<=r} g_s (per key channel), P_r = e^{G_r}, Gam = e^{G_15}:
//   Kt = k * P,  Qt = q * P,  Kc = k / P,  Ke = k * Gam / P
//   A[r,i] = b_r <Kt_r, Kc_i>  (i < r),   M[r,i] = <Qt_r, Kc_i>  (i <= r)
//   T      = (I + A)^{-1} Diag(b)
//   U      = T (V - Kt S)
//   O      = Qt S + M U
//   S_out  = Diag(Gam) S + Ke^T U
// With the chunk start as the reference point every factor spans at most 16
// positions: P and Gam / P lie in [e^-80, 1] and 1 / P in [1, e^80] -- exactly
// the range the pages' bound guarantees.  Every factor is built as a running
// product of a_t = exp(g_t) (one exponential per element).
//
// Work decomposition.  A workgroup owns one (sequence, head, 64-wide value
// slice); value columns of S never interact.  It runs 8 wavefronts:
//   consumers 0..3  -- wavefront w keeps value columns [16w, 16w+16) of the
//                      dk x 64 fp32 state in MFMA accumulators for the whole
//                      sequence and runs the state-dependent products of every
//                      chunk in order; o goes straight to HBM;
//   producers 4..7  -- producer p owns chunks p, p+4, p+8, ...: it loads them
//                      (one chunk of prefetch in registers), builds the decayed
//                      operands with in-register running products (lane = two
//                      key channels, registers = the 16 tokens), forms A and M
//                      on MFMA, inverts I + A by forward substitution and
//                      publishes everything in a ring of NS LDS slots.
// Producers and consumers hand slots over through per-slot LDS flags ("ready"
// and per-consumer "done"); every wait is bounded and a WG-wide abort flag ends
// all waits if one ever runs out (the result is then wrong, never a hang).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kWsThreads = 512;
constexpr int kC = 16;                 // tokens per chunk
constexpr int kVS = 64;                // value columns per workgroup
constexpr int kXCDs = 8;
constexpr int kSpinLimit = 1 << 22;

template <typename E, int DK>
struct WsL {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int NS = ES == 2 ? 8 : 3;        // LDS slots
    static constexpr int LDK = DK + 16 / ES;          // padded row of [16][DK]
    static constexpr int LT = 16;                     // row of [*][16]
    // slot, E-typed part (element offsets)
    static constexpr int eKt = 0;                     // Kt   [16][LDK]  token-major
    static constexpr int eQt = eKt + kC * LDK;        // Qt   [16][LDK]
    static constexpr int eKeT = eQt + kC * LDK;       // Ke^T [DK][16]   channel-major
    static constexpr int eVT = eKeT + DK * LT;        // V^T  [64][16]
    static constexpr int eT = eVT + kVS * LT;         // T    [16][16]
    static constexpr int eM = eT + kC * LT;           // M    [16][16]
    static constexpr int slotE = eM + kC * LT;
    static constexpr int slotBytes = slotE * ES + DK * 4;   // + Gam fp32 [DK]
    // producer scratch
    static constexpr int pKc = 0;                     // Kc [16][LDK] token-major (E)
    static constexpr int pBytesE = kC * LDK * ES;
    static constexpr int LA = 20;                     // row of A (16-byte aligned)
    static constexpr int pA = 0;                      // A  [16][LA] fp32
    static constexpr int pBeta = 16 * LA;             // beta [16] fp32
    static constexpr int pBytes = pBytesE + (pBeta + 16) * 4;
    // byte offsets
    static constexpr int oSlots = 0;
    static constexpr int oProd = oSlots + NS * slotBytes;
    static constexpr int oFlags = oProd + 4 * pBytes;
    static constexpr int nFlags = NS + NS * 4 + 1;    // ready[NS], done[NS][4], abort
    static constexpr int bytes = oFlags + nFlags * 4;
    static_assert(slotBytes % 16 == 0 && pBytesE % 16 == 0 && pBytes % 16 == 0, "alignment");
};

__device__ __forceinline__ void lds_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup"); }

__device__ __forceinline__ int ld_flag(const int *f)
{
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void st_flag(int *f, int v)
{
    __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wait until every flag f[i * stride], i < n, is >= target.  Bounded: after
// kSpinLimit polls the WG abort flag is raised and all later waits return.
__device__ __forceinline__ void wait_flags(const int *f, int n, int stride, int target, int *abort_flag)
{
    int spins = 0;
    for (;;) {
        bool ok = true;
        for (int i = 0; i < n; ++i)
            ok = ok && ld_flag(f + i * stride) >= target;
        if (ok || ld_flag(abort_flag))
            break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
            st_flag(abort_flag, 1);
            break;
        }
    }
    lds_fence();
}

// Two adjacent elements as one register-sized pack.
template <typename E> struct Pair;
template <> struct Pair<__bf16> {
    typedef unsigned int T;
    static __device__ __forceinline__ float lo(T x) { return __uint_as_float(x << 16); }
    static __device__ __forceinline__ float hi(T x) { return __uint_as_float(x & 0xffff0000u); }
    static __device__ __forceinline__ T pack(float a, float b)
    {
        typedef __bf16 v2 __attribute__((ext_vector_type(2)));
        v2 r;
        r[0] = (__bf16)a;
        r[1] = (__bf16)b;
        return __builtin_bit_cast(T, r);
    }
    static __device__ __forceinline__ T zero() { return 0u; }
};
template <> struct Pair<float> {
    typedef float2 T;
    static __device__ __forceinline__ float lo(T x) { return x.x; }
    static __device__ __forceinline__ float hi(T x) { return x.y; }
    static __device__ __forceinline__ T pack(float a, float b) { return make_float2(a, b); }
    static __device__ __forceinline__ T zero() { return make_float2(0.f, 0.f); }
};

// One chunk's raw inputs for one producer wave: lane l holds key channels
// 2l, 2l+1 of q, k, g for the 16 tokens, value columns 2l, 2l+1 of the slice
// (lanes < 32) and beta of token l (lanes < 16).
template <typename E>
struct Raw {
    typename Pair<E>::T q[kC], k[kC], g[kC], v[kC];
    E b;
};

template <typename E, int DK>
__device__ __forceinline__ void load_raw(Raw<E> &R, const E *qh, const E *kh, const E *gh,
                                         const E *vh, const E *bh, long tok0, int valid, int H,
                                         int DV, int slice, int lane)
{
    typedef Pair<E> PE;
    typedef typename PE::T PT;
    const bool kch = 2 * lane < DK, vch = lane < kVS / 2;
#pragma unroll
    for (int r = 0; r < kC; ++r) {
        R.q[r] = R.k[r] = R.g[r] = R.v[r] = PE::zero();
        if (r < valid) {
            const long row = (tok0 + r) * H;
            if (kch) {
                R.q[r] = *reinterpret_cast<const PT *>(qh + row * DK + 2 * lane);
                R.k[r] = *reinterpret_cast<const PT *>(kh + row * DK + 2 * lane);
                R.g[r] = *reinterpret_cast<const PT *>(gh + row * DK + 2 * lane);
            }
            if (vch)
                R.v[r] = *reinterpret_cast<const PT *>(vh + row * DV + slice * kVS + 2 * lane);
        }
    }
    R.b = from_f<E>(0.f);
    if (lane < valid && lane < kC)
        R.b = bh[(tok0 + lane) * H];
}

template <typename E, int DK>
__global__ __launch_bounds__(kWsThreads) void prefill_ws_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const E *__restrict__ g, const E *__restrict__ beta, const float *S0, E *__restrict__ o,
    float *S_T, int T, int H, int DV, int nbh, int nsl)
{
    typedef WsL<E, DK> L;
    typedef typename Vec<E>::v4 V4;
    typedef typename Vec<E>::v8 V8;
    typedef Pair<E> PE;
    constexpr int NS = L::NS;
    constexpr int NCT = DK / 16, NKS = DK / 32;

    extern __shared__ __align__(16) unsigned char smem[];
    int *flags = reinterpret_cast<int *>(smem + L::oFlags);
    int *ready = flags;                 // [NS]
    int *done = flags + NS;             // [NS][4]
    int *abort_flag = flags + NS + 4 * NS;

    // workgroup -> (head, value slice); slices of a head share an XCD's L2
    const int id = blockIdx.x, xcd = id % kXCDs, rr = id / kXCDs;
    const int bh = (rr / nsl) * kXCDs + xcd, slice = rr % nsl;
    if (bh >= nbh)
        return;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const long tokb = (long)b * T;
    const int nchunks = (T + kC - 1) / kC;

    for (int i = tid; i < L::nFlags; i += kWsThreads)
        flags[i] = 0;
    __syncthreads();

    if (wave < 4) {
        // =============================== consumer ===============================
        const int w = wave;
        const int col = slice * kVS + 16 * w + l16;      // this lane's value column
        f32x4 Sacc[NCT];                                  // S[16 ct + 4 g4 + j][col]
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Sacc[ct][j] = S0 ? S0[((long)bh * DK + 16 * ct + 4 * g4 + j) * DV + col] : 0.f;
        E *oh = o + (long)h * DV + col;

        for (int c = 0; c < nchunks; ++c) {
            const int s = c % NS;
            // S strip as B operands; contraction slice m holds channels
            // {32m + 4 g4 + e, 32m + 16 + 4 g4 + e}, e = 0..3
            V8 Bs[NKS];
#pragma unroll
            for (int m = 0; m < NKS; ++m)
                Bs[m] = cat8(cvt4<E>(Sacc[2 * m]), cvt4<E>(Sacc[2 * m + 1]));

            wait_flags(ready + s, 1, 1, c + 1, abort_flag);
            const E *sl = reinterpret_cast<const E *>(smem + L::oSlots + s * L::slotBytes);
            const float *gam = reinterpret_cast<const float *>(smem + L::oSlots + s * L::slotBytes + L::slotE * L::ES);

            f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
            const E *kt = sl + L::eKt + l16 * L::LDK + 4 * g4;
            const E *qt = sl + L::eQt + l16 * L::LDK + 4 * g4;
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                const V8 a = cat8(*reinterpret_cast<const V4 *>(kt + 32 * m),
                                  *reinterpret_cast<const V4 *>(kt + 32 * m + 16));
                const V8 aq = cat8(*reinterpret_cast<const V4 *>(qt + 32 * m),
                                   *reinterpret_cast<const V4 *>(qt + 32 * m + 16));
                X = mma32(a, Bs[m], X);
                Y = mma32(aq, Bs[m], Y);
            }
            // X <- V - Kt S   (rows 4 g4 + j = tokens, column l16)
            const V4 vv = *reinterpret_cast<const V4 *>(sl + L::eVT + (16 * w + l16) * L::LT + 4 * g4);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                X[j] = to_f(vv[j]) - X[j];
            // U = T X, then O = Y + M U   (contraction over tokens 4 g4 + e)
            const V4 tr = *reinterpret_cast<const V4 *>(sl + L::eT + l16 * L::LT + 4 * g4);
            const f32x4 U = mma16(tr, cvt4<E>(X), f32x4{0.f, 0.f, 0.f, 0.f});
            const V4 bu = cvt4<E>(U);
            const V4 mr = *reinterpret_cast<const V4 *>(sl + L::eM + l16 * L::LT + 4 * g4);
            const f32x4 Z = mma16(mr, bu, f32x4{0.f, 0.f, 0.f, 0.f});
            // S <- Gam S + Ke^T U
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const V4 kr = *reinterpret_cast<const V4 *>(sl + L::eKeT + (16 * ct + l16) * L::LT + 4 * g4);
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(gam + 16 * ct + 4 * g4);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    Sacc[ct][j] *= gm[j];
                Sacc[ct] = mma16(kr, bu, Sacc[ct]);
            }
            // every read of slot s has landed in registers: hand it back
            lds_fence();
            if (lane == 0)
                st_flag(done + s * 4 + w, c + 1);
            // o rows of this chunk
            const int t0 = c * kC;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * g4 + j;
                if (t0 + r < T)
                    oh[((tokb + t0 + r) * H) * (long)DV] = from_f<E>(Y[j] + Z[j]);
            }
        }
        if (S_T) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    S_T[((long)bh * DK + 16 * ct + 4 * g4 + j) * DV + col] = Sacc[ct][j];
        }
        return;
    }

    // ================================= producer =================================
    const int pw = wave - 4;
    unsigned char *pscr = smem + L::oProd + pw * L::pBytes;
    E *pKc = reinterpret_cast<E *>(pscr);
    float *pA = reinterpret_cast<float *>(pscr + L::pBytesE);
    float *pBeta = pA + L::pBeta;
    const E *qh = q + (long)h * DK, *kh = k + (long)h * DK, *gh = g + (long)h * DK;
    const E *vh = v + (long)h * DV, *bh_ = beta + h;
    const bool kch = 2 * lane < DK, vch = lane < kVS / 2;
    const float kLog2e = 1.4426950408889634f;

    // bf16: one chunk of register prefetch (issued a whole producer round
    // ahead); fp32 test mode loads on demand (its registers are twice as big)
    constexpr bool kPrefetch = sizeof(E) == 2;
    Raw<E> nxt;
    if (kPrefetch && pw < nchunks) {
        const int t0 = pw * kC;
        load_raw<E, DK>(nxt, qh, kh, gh, vh, bh_, tokb + t0, T - t0 < kC ? T - t0 : kC, H, DV, slice, lane);
    }
    for (int c = pw; c < nchunks; c += 4) {
        Raw<E> cur;
        if (kPrefetch) {
            cur = nxt;
            if (c + 4 < nchunks) {
                const int t1 = (c + 4) * kC;
                load_raw<E, DK>(nxt, qh, kh, gh, vh, bh_, tokb + t1, T - t1 < kC ? T - t1 : kC, H, DV, slice, lane);
            }
        } else {
            const int t0 = c * kC;
            load_raw<E, DK>(cur, qh, kh, gh, vh, bh_, tokb + t0, T - t0 < kC ? T - t0 : kC, H, DV, slice, lane);
        }
        const int s = c % NS;
        if (c >= NS)
            wait_flags(done + s * 4, 4, 1, c - NS + 1, abort_flag);
        E *sl = reinterpret_cast<E *>(smem + L::oSlots + s * L::slotBytes);
        float *gam = reinterpret_cast<float *>(smem + L::oSlots + s * L::slotBytes + L::slotE * L::ES);

        // ---- decay factors by running products, then the operands ------------
        if (kch) {
            float a0[kC], a1[kC];
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                a0[r] = __builtin_amdgcn_exp2f(PE::lo(cur.g[r]) * kLog2e);
                a1[r] = __builtin_amdgcn_exp2f(PE::hi(cur.g[r]) * kLog2e);
            }
            float P0[kC], P1[kC], Z0[kC], Z1[kC];       // prefix e^{G_r}, suffix e^{G_15 - G_r}
            float p0 = 1.f, p1 = 1.f;
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                p0 *= a0[r];
                p1 *= a1[r];
                P0[r] = p0;
                P1[r] = p1;
            }
            float z0 = 1.f, z1 = 1.f;
#pragma unroll
            for (int r = kC - 1; r >= 0; --r) {
                Z0[r] = z0;
                Z1[r] = z1;
                z0 *= a0[r];
                z1 *= a1[r];
            }
            const float ig0 = 1.f / p0, ig1 = 1.f / p1;  // 1 / Gam
            *reinterpret_cast<float2 *>(gam + 2 * lane) = make_float2(p0, p1);
            float ke0[kC], ke1[kC];
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                const float k0 = PE::lo(cur.k[r]), k1 = PE::hi(cur.k[r]);
                const float q0 = PE::lo(cur.q[r]), q1 = PE::hi(cur.q[r]);
                const float ip0 = Z0[r] * ig0, ip1 = Z1[r] * ig1;   // 1 / P_r
                *reinterpret_cast<typename PE::T *>(sl + L::eKt + r * L::LDK + 2 * lane) = PE::pack(k0 * P0[r], k1 * P1[r]);
                *reinterpret_cast<typename PE::T *>(sl + L::eQt + r * L::LDK + 2 * lane) = PE::pack(q0 * P0[r], q1 * P1[r]);
                *reinterpret_cast<typename PE::T *>(pKc + r * L::LDK + 2 * lane) = PE::pack(k0 * ip0, k1 * ip1);
                ke0[r] = k0 * Z0[r];          // Ke = k Gam / P = k * suffix product
                ke1[r] = k1 * Z1[r];
            }
            // channel-major rows: the 16 tokens of channel 2l, then of 2l+1
            E *r0 = sl + L::eKeT + (2 * lane) * L::LT;
            E *r1 = r0 + L::LT;
#pragma unroll
            for (int r = 0; r < kC; r += 2) {
                *reinterpret_cast<typename PE::T *>(r0 + r) = PE::pack(ke0[r], ke0[r + 1]);
                *reinterpret_cast<typename PE::T *>(r1 + r) = PE::pack(ke1[r], ke1[r + 1]);
            }
        }
        if (vch) {
            E *r0 = sl + L::eVT + (2 * lane) * L::LT;
            E *r1 = r0 + L::LT;
#pragma unroll
            for (int r = 0; r < kC; r += 2) {
                *reinterpret_cast<typename PE::T *>(r0 + r) = PE::pack(PE::lo(cur.v[r]), PE::lo(cur.v[r + 1]));
                *reinterpret_cast<typename PE::T *>(r1 + r) = PE::pack(PE::hi(cur.v[r]), PE::hi(cur.v[r + 1]));
            }
        }
        if (lane < kC)
            pBeta[lane] = to_f(cur.b);
        lds_fence();

        // ---- A and M on MFMA (contraction over the DK channels) ----------------
        {
            f32x4 Aacc = {0.f, 0.f, 0.f, 0.f}, Macc = {0.f, 0.f, 0.f, 0.f};
            const E *kt = sl + L::eKt + l16 * L::LDK + 8 * g4;
            const E *qt = sl + L::eQt + l16 * L::LDK + 8 * g4;
            const E *kc = pKc + l16 * L::LDK + 8 * g4;
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                const V8 ak = cat8(*reinterpret_cast<const V4 *>(kt + 32 * m), *reinterpret_cast<const V4 *>(kt + 32 * m + 4));
                const V8 aq = cat8(*reinterpret_cast<const V4 *>(qt + 32 * m), *reinterpret_cast<const V4 *>(qt + 32 * m + 4));
                const V8 bc = cat8(*reinterpret_cast<const V4 *>(kc + 32 * m), *reinterpret_cast<const V4 *>(kc + 32 * m + 4));
                Aacc = mma32(ak, bc, Aacc);
                Macc = mma32(aq, bc, Macc);
            }
            // lane holds rows 4 g4 + j, column l16
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * g4 + j, i = l16;
                pA[r * L::LA + i] = i < r ? pBeta[r] * Aacc[j] : 0.f;
                sl[L::eM + r * L::LT + i] = from_f<E>(i <= r ? Macc[j] : 0.f);
            }
        }
        lds_fence();

        // ---- T = (I + A)^{-1} Diag(beta): forward substitution, lane = column l16
        {
            const int j = l16;
            float x[kC];
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4 *>(pA + r * L::LA + 4 * i4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * i4 + e < r)
                            acc -= a4[e] * x[4 * i4 + e];
                }
                x[r] = acc;
            }
            const float bj = pBeta[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                sl[L::eT + r * L::LT + j] = from_f<E>(x[r] * bj);
            }
        }
        // publish the slot
        lds_fence();
        if (lane == 0)
            st_flag(ready + s, c + 1);
    }
}

template <typename E, int DK>
hipError_t launch_ws(const void *q, const void *k, const void *v, const void *g, const void *beta,
                     const float *S0, void *o, float *S_T, int B, int T, int H, int dv,
                     hipStream_t stream)
{
    typedef WsL<E, DK> L;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    constexpr int lds = L::bytes > 81 * 1024 ? L::bytes : 81 * 1024;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)prefill_ws_kernel<E, DK>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    const int nbh = B * H, nsl = dv / kVS;
    const int grid = ((nbh + kXCDs - 1) / kXCDs) * kXCDs * nsl;
    hipLaunchKernelGGL((prefill_ws_kernel<E, DK>), dim3(grid), dim3(kWsThreads), lds, stream,
                       (const E *)q, (const E *)k, (const E *)v, (const E *)g, (const E *)beta, S0,
                       (E *)o, S_T, T, H, dv, nbh, nsl);
    return hipGetLastError();
}

} // namespace

hipError_t launch_chunk16(const void *q, const void *k, const void *v, const void *g,
                          const void *beta, const float *S0, void *o, float *S_T, int B, int T,
                          int H, int dk, int dv, bool fp32, hipStream_t stream)
{
    if (fp32)
        return dk == 128 ? launch_ws<float, 128>(q, k, v, g, beta, S0, o, S_T, B, T, H, dv, stream)
                         : launch_ws<float, 64>(q, k, v, g, beta, S0, o, S_T, B, T, H, dv, stream);
    return dk == 128 ? launch_ws<__bf16, 128>(q, k, v, g, beta, S0, o, S_T, B, T, H, dv, stream)
                     : launch_ws<__bf16, 64>(q, k, v, g, beta, S0, o, S_T, B, T, H, dv, stream);
}

} // namespace kda
