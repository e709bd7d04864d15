// kda_bwd.hip -- backward pass of the KDA recurrence on gfx950 (kda_chunk_bwd).
//
// Method: page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section 3.3:
// training runs the chunked form (X_[c], S_in) -> (Y_[c], S_out) with
// S_in(c+1) = S_out(c) of the recurrence of section 3.1.  The pages derive no
// backward pass; this file computes the exact reverse mode of that chunk map.
// Per chunk of n <= 16 tokens with incoming state S, chunk-relative cumulative
// log-decay G (per key channel), P = e^G and Gam = P[n-1]:
//   forward  Kt = k P, Qt = q P, Kc = k / P, Ke = k Gam / P,  B = Kt Kc^T,
//            A = strict_lower(Diag(beta) B), L = (I + A)^{-1}, Tm = L Diag(beta),
//            X = V - Kt S, U = Tm X, M = lower(Qt Kc^T),
//            O = Qt S + M U,  S' = Diag(Gam) S + Ke^T U;
//   reverse  given dO and D = dLoss/dS':
//            dU = M^T dO + Ke D,  dX = Tm^T dU,  dV = dX,
//            dM = lower(dO U^T),  dTm = dU X^T,  dL = dTm Diag(beta),
//            dA = strict_lower(-L^T dL L^T),  dB = Diag(beta) dA,
//            dbeta_i = sum_r L[r,i] dTm[r,i] + sum_{j<i} dA[i,j] B[i,j],
//            dQt = dO S^T + dM Kc,  dKe = U D^T,
//            dKt = -dX S^T + dB Kc,  dKc = dM^T Qt + dB^T Kt,
//            dG  = dKt Kt + dQt Qt - dKc Kc - dKe Ke  (+ on the last token
//                  rowsum(D (.) S) Gam + sum_r dKe Ke),
//            dq = dQt P,  dk = dKt P + dKc / P + dKe Gam / P,
//            dg = reverse cumulative sum of dG over the chunk's tokens,
//            D_in = Diag(Gam) D + Qt^T dO - Kt^T dX.
// A forward pass (the chunk-16 prefill kernel writing its state after every
// chunk) supplies each chunk's incoming state S.
//
// Work decomposition: one workgroup of 256 threads per (sequence, head,
// 64-wide value slice) walks the chunks from last to first.  The slice's part
// of D lives in LDS for the whole walk, the slice's part of S is loaded per
// chunk; every product is an fp32 FMA loop from LDS.  dV and dS0 are per value
// column and written directly.  dq, dk, dg and dbeta are sums over all value
// columns, and every expression above after the column contractions (dM, dTm,
// dQt, dKe, dKt and rowsum(D S)) is linear in them, so each slice computes the
// whole chain on its own columns and writes a partial; a second kernel adds
// the slices' partials in slice order (no atomics: the result is
// deterministic).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kBT = 256;        // threads per workgroup
constexpr int kNV = 64;         // value columns per workgroup
constexpr int kC = 16;          // tokens per chunk
constexpr int kXCDs = 8;

template <int DK>
struct BwdL {
    static constexpr int SS = kNV + 1;          // row stride of S and D  [DK][SS]
    static constexpr int OS = DK + 1;           // row stride of [16][DK] operand arrays
    static constexpr int CS = kNV + 1;          // row stride of [16][NV] column arrays
    static constexpr int MS = kC + 1;           // row stride of [16][16] matrices
    static constexpr int oS = 0;
    static constexpr int oD = oS + DK * SS;
    static constexpr int oKt = oD + DK * SS;
    static constexpr int oQt = oKt + kC * OS;
    static constexpr int oKc = oQt + kC * OS;
    static constexpr int oKe = oKc + kC * OS;
    static constexpr int oP = oKe + kC * OS;
    static constexpr int oT1 = oP + kC * OS;    // staging: dG
    static constexpr int oT2 = oT1 + kC * OS;   // staging: dKe * Ke
    static constexpr int oX = oT2 + kC * OS;    // V, then X
    static constexpr int oU = oX + kC * CS;
    static constexpr int oDO = oU + kC * CS;
    static constexpr int oDU = oDO + kC * CS;
    static constexpr int oDX = oDU + kC * CS;
    static constexpr int oB = oDX + kC * CS;    // B = Kt Kc^T
    static constexpr int oL = oB + kC * MS;     // L = (I + A)^{-1}
    static constexpr int oTm = oL + kC * MS;    // Tm = L Diag(beta)
    static constexpr int oM = oTm + kC * MS;    // M = lower(Qt Kc^T)
    static constexpr int oDM = oM + kC * MS;    // dM
    static constexpr int oDT = oDM + kC * MS;   // dTm, then dL L^T
    static constexpr int oDB = oDT + kC * MS;   // dB
    static constexpr int oGam = oDB + kC * MS;  // Gam [DK]
    static constexpr int oGd = oGam + DK;       // rowsum(D S) [DK]
    static constexpr int oBeta = oGd + DK;      // beta [16]
    static constexpr int floats = oBeta + kC;
    static constexpr int bytes = floats * 4;
};

__device__ __forceinline__ float ldE(const __bf16 *p) { return (float)*p; }
__device__ __forceinline__ float ldE(const float *p) { return *p; }

template <typename E, int DK>
__global__ __launch_bounds__(kBT) void bwd_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v, const E *__restrict__ g,
    const E *__restrict__ beta, const float *__restrict__ S0, const E *__restrict__ dO,
    const float *__restrict__ dST, const float *__restrict__ states, float *__restrict__ dv_out,
    float *__restrict__ dS0_out, float *__restrict__ pq, float *__restrict__ pk, float *__restrict__ pg,
    float *__restrict__ pb, int T, int H, int DV, int nbh, int nsl)
{
    typedef BwdL<DK> L;
    extern __shared__ __align__(16) float sm[];
    float *Ss = sm + L::oS, *Ds = sm + L::oD;
    float *Kt = sm + L::oKt, *Qt = sm + L::oQt, *Kc = sm + L::oKc, *Ke = sm + L::oKe, *Pm = sm + L::oP;
    float *T1 = sm + L::oT1, *T2 = sm + L::oT2;
    float *Xs = sm + L::oX, *Us = sm + L::oU, *dOs = sm + L::oDO, *dUs = sm + L::oDU, *dXs = sm + L::oDX;
    float *Bm = sm + L::oB, *Lm = sm + L::oL, *Tm = sm + L::oTm, *Mm = sm + L::oM;
    float *dM = sm + L::oDM, *dT = sm + L::oDT, *dB = sm + L::oDB;
    float *Gam = sm + L::oGam, *Gd = sm + L::oGd, *bet = sm + L::oBeta;

    // workgroup -> (head, value slice); slices of a head share an XCD's L2
    const int id = blockIdx.x, xcd = id % kXCDs, rr = id / kXCDs;
    const int bh = (rr / nsl) * kXCDs + xcd, slice = rr % nsl;
    if (bh >= nbh)
        return;
    const int b = bh / H, h = bh % H;
    const int t = threadIdx.x;
    const int col0 = slice * kNV;
    const long tokb = (long)b * T;
    const int nchunks = (T + kC - 1) / kC;
    const long sbase = (long)bh * DK * DV;                 // this head's state in [B,H,DK,DV]

    // D <- dS_T (slice columns)
    for (int e = t; e < DK * kNV; e += kBT) {
        const int c = e / kNV, j = e % kNV;
        Ds[c * L::SS + j] = dST ? dST[sbase + (long)c * DV + col0 + j] : 0.f;
    }

    for (int ci = nchunks - 1; ci >= 0; --ci) {
        const int t0 = ci * kC;
        const int n = T - t0 < kC ? T - t0 : kC;
        __syncthreads();   // previous chunk's readers of every array are done
        // ---- the chunk's incoming state and inputs --------------------------------
        const float *Sin = ci == 0 ? (S0 ? S0 + sbase : nullptr)
                                   : states + (long)(ci - 1) * nbh * DK * DV + sbase;
        for (int e = t; e < DK * kNV; e += kBT) {
            const int c = e / kNV, j = e % kNV;
            Ss[c * L::SS + j] = Sin ? Sin[(long)c * DV + col0 + j] : 0.f;
        }
        // q, k as Qt, Kt (scaled below), g into Pm; rows r >= n are zero
        for (int e = t; e < kC * DK; e += kBT) {
            const int r = e / DK, c = e % DK;
            const long off = ((tokb + t0 + r) * H + h) * DK + c;
            const bool ok = r < n;
            Qt[r * L::OS + c] = ok ? ldE(q + off) : 0.f;
            Kt[r * L::OS + c] = ok ? ldE(k + off) : 0.f;
            Pm[r * L::OS + c] = ok ? ldE(g + off) : 0.f;
        }
        for (int e = t; e < kC * kNV; e += kBT) {
            const int r = e / kNV, j = e % kNV;
            const long off = ((tokb + t0 + r) * H + h) * (long)DV + col0 + j;
            const bool ok = r < n;
            Xs[r * L::CS + j] = ok ? ldE(v + off) : 0.f;
            dOs[r * L::CS + j] = ok ? ldE(dO + off) : 0.f;
        }
        if (t < kC)
            bet[t] = t < n ? ldE(beta + (tokb + t0 + t) * H + h) : 0.f;
        __syncthreads();

        // ---- decay factors and operands (thread per key channel) ---------------
        if (t < DK) {
            const int c = t;
            float G = 0.f;
            for (int r = 0; r < kC; ++r) {
                G += Pm[r * L::OS + c];                   // g (0 past the last token)
                Pm[r * L::OS + c] = exp_f(G);
            }
            const float gm = Pm[(n - 1) * L::OS + c];
            Gam[c] = gm;
            for (int r = 0; r < kC; ++r) {
                const float p = Pm[r * L::OS + c], kk = Kt[r * L::OS + c], qq = Qt[r * L::OS + c];
                const float ip = 1.0f / p;
                Kt[r * L::OS + c] = kk * p;
                Qt[r * L::OS + c] = qq * p;
                Kc[r * L::OS + c] = kk * ip;
                Ke[r * L::OS + c] = kk * (gm * ip);
            }
        }
        __syncthreads();

        // ---- B = Kt Kc^T and M = lower(Qt Kc^T) (thread per entry) --------------
        {
            const int r = t >> 4, i = t & 15;
            float sb = 0.f, sq = 0.f;
#pragma unroll 8
            for (int c = 0; c < DK; ++c) {
                const float kc = Kc[i * L::OS + c];
                sb += Kt[r * L::OS + c] * kc;
                sq += Qt[r * L::OS + c] * kc;
            }
            Bm[r * L::MS + i] = sb;
            Mm[r * L::MS + i] = i <= r ? sq : 0.f;
        }
        __syncthreads();
        // ---- L = (I + A)^{-1} by forward substitution (thread per column) -------
        if (t < kC) {
            const int i = t;
            float col[kC];
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                float x = r == i ? 1.f : 0.f;
                const float br = bet[r];
#pragma unroll
                for (int j = 0; j < r; ++j)
                    x -= br * Bm[r * L::MS + j] * col[j];
                col[r] = x;
            }
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                Lm[r * L::MS + i] = col[r];
                Tm[r * L::MS + i] = col[r] * bet[i];
            }
        }
        __syncthreads();

        // ---- column products: thread (r, 4 columns j = jj + 16 u) ---------------
        const int r4 = t >> 4, jj = t & 15;
        {
            // X = V - Kt S
            float a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                a[u] = Xs[r4 * L::CS + jj + 16 * u];
#pragma unroll 8
            for (int c = 0; c < DK; ++c) {
                const float kt = Kt[r4 * L::OS + c];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    a[u] -= kt * Ss[c * L::SS + jj + 16 * u];
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 4; ++u)
                Xs[r4 * L::CS + jj + 16 * u] = a[u];
        }
        __syncthreads();
        {
            // U = Tm X;  dU = M^T dO + Ke D
            float uu[4] = {0.f, 0.f, 0.f, 0.f}, du[4] = {0.f, 0.f, 0.f, 0.f};
            for (int i = 0; i < kC; ++i) {
                const float tm = Tm[r4 * L::MS + i], mt = Mm[i * L::MS + r4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    uu[u] += tm * Xs[i * L::CS + jj + 16 * u];
                    du[u] += mt * dOs[i * L::CS + jj + 16 * u];
                }
            }
#pragma unroll 8
            for (int c = 0; c < DK; ++c) {
                const float ke = Ke[r4 * L::OS + c];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    du[u] += ke * Ds[c * L::SS + jj + 16 * u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                Us[r4 * L::CS + jj + 16 * u] = uu[u];
                dUs[r4 * L::CS + jj + 16 * u] = du[u];
            }
        }
        __syncthreads();
        {
            // dX = Tm^T dU = dV
            float dx[4] = {0.f, 0.f, 0.f, 0.f};
            for (int i = 0; i < kC; ++i) {
                const float tm = Tm[i * L::MS + r4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    dx[u] += tm * dUs[i * L::CS + jj + 16 * u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                dXs[r4 * L::CS + jj + 16 * u] = dx[u];
                if (r4 < n)
                    dv_out[((tokb + t0 + r4) * H + h) * (long)DV + col0 + jj + 16 * u] = dx[u];
            }
        }
        // dM = lower(dO U^T), dTm = dU X^T over this slice's columns
        {
            const int r = t >> 4, i = t & 15;
            float sm_ = 0.f, st = 0.f;
#pragma unroll 8
            for (int j = 0; j < kNV; ++j) {
                sm_ += dOs[r * L::CS + j] * Us[i * L::CS + j];
                st += dUs[r * L::CS + j] * Xs[i * L::CS + j];
            }
            __syncthreads();   // dX written by every thread before it is read below
            dM[r * L::MS + i] = i <= r ? sm_ : 0.f;
            dT[r * L::MS + i] = st;
        }
        __syncthreads();
        // dbeta (direct part) and W = dL L^T with dL = dTm Diag(beta), in place of dTm
        {
            const int r = t >> 4, i = t & 15;
            float w = 0.f;
            for (int j = 0; j < kC; ++j)
                w += dT[r * L::MS + j] * bet[j] * Lm[i * L::MS + j];
            float dbd = 0.f;
            if (t < kC)
                for (int rr2 = 0; rr2 < kC; ++rr2)
                    dbd += Lm[rr2 * L::MS + t] * dT[rr2 * L::MS + t];
            __syncthreads();
            dT[r * L::MS + i] = w;
            if (t < kC)
                Gd[t] = dbd;          // temporary: direct dbeta (Gd is filled later)
        }
        __syncthreads();
        // dA = strict_lower(-L^T W), dB = Diag(beta) dA, dbeta += sum_{i<r} dA B
        {
            const int r = t >> 4, i = t & 15;
            float a = 0.f;
            if (i < r)
                for (int j = 0; j < kC; ++j)
                    a -= Lm[j * L::MS + r] * dT[j * L::MS + i];
            dB[r * L::MS + i] = bet[r] * a;
            float prod = a * Bm[r * L::MS + i];
            // reduce prod over the 16 lanes i of row r (xor shuffles stay in the row)
#pragma unroll
            for (int off = 8; off > 0; off >>= 1)
                prod += __shfl_xor(prod, off, 64);
            if (i == 0)
                T2[r] = prod;         // temporary: dbeta from A
        }
        __syncthreads();
        if (t < kC && t < n) {
            const long bo = (long)slice * ((long)nbh / H * T * H) + (tokb + t0 + t) * H + h;
            pb[bo] = Gd[t] + T2[t];
        }
        __syncthreads();

        // ---- parameter gradients: thread (r, channels c = cc + 16 u) ----------------
        {
            const int r = t >> 4, cc = t & 15;
            const long row = (tokb + t0 + r) * H + h;
            const long so = (long)slice * ((long)nbh / H * T * H) * DK;
#pragma unroll 1
            for (int u = 0; u < DK / 16; ++u) {
                const int c = cc + 16 * u;
                float qt = 0.f, ke = 0.f, ktt = 0.f, kcc = 0.f;
#pragma unroll 8
                for (int j = 0; j < kNV; ++j) {
                    const float s = Ss[c * L::SS + j];
                    qt += dOs[r * L::CS + j] * s;
                    ktt -= dXs[r * L::CS + j] * s;
                    ke += Us[r * L::CS + j] * Ds[c * L::SS + j];
                }
                for (int i = 0; i < kC; ++i) {
                    const float kci = Kc[i * L::OS + c];
                    qt += dM[r * L::MS + i] * kci;
                    ktt += dB[r * L::MS + i] * kci;
                    kcc += dM[i * L::MS + r] * Qt[i * L::OS + c] + dB[i * L::MS + r] * Kt[i * L::OS + c];
                }
                const float p = Pm[r * L::OS + c], ip = 1.0f / p, gm = Gam[c];
                const float keke = ke * Ke[r * L::OS + c];
                if (r < n) {
                    pq[so + row * DK + c] = qt * p;
                    pk[so + row * DK + c] = ktt * p + kcc * ip + ke * (gm * ip);
                }
                T1[r * L::OS + c] = ktt * Kt[r * L::OS + c] + qt * Qt[r * L::OS + c] - kcc * Kc[r * L::OS + c] - keke;
                T2[r * L::OS + c] = keke;
            }
        }
        // rowsum(D (.) S) per key channel
        if (t < DK) {
            float s = 0.f;
#pragma unroll 8
            for (int j = 0; j < kNV; ++j)
                s += Ds[t * L::SS + j] * Ss[t * L::SS + j];
            Gd[t] = s;
        }
        __syncthreads();
        // dg: the last token's extra terms, then a reverse cumulative sum
        if (t < DK) {
            const int c = t;
            float extra = Gd[c] * Gam[c];
            for (int r = 0; r < kC; ++r)
                extra += T2[r * L::OS + c];
            float acc = 0.f;
            const long so = (long)slice * ((long)nbh / H * T * H) * DK;
            for (int r = n - 1; r >= 0; --r) {
                acc += T1[r * L::OS + c] + (r == n - 1 ? extra : 0.f);
                pg[so + ((tokb + t0 + r) * H + h) * DK + c] = acc;
            }
        }
        __syncthreads();

        // ---- D <- Diag(Gam) D + Qt^T dO - Kt^T dX: thread owns 4 rows x 8 columns ----
        // 32 row blocks of 4 x 8 column blocks of 8 cover 128 rows x 64 columns
        // (with dk = 64 the upper half of the row blocks has no rows)
        {
            const int cb = t >> 3, jb = t & 7;
            const int c0 = 4 * cb;
            if (c0 < DK) {
                float acc[4][8];
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[a][j] = Gam[c0 + a] * Ds[(c0 + a) * L::SS + 8 * jb + j];
#pragma unroll 2
                for (int r = 0; r < kC; ++r) {
                    float qa[4], ka[4], dov[8], dxv[8];
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        qa[a] = Qt[r * L::OS + c0 + a];
                        ka[a] = Kt[r * L::OS + c0 + a];
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        dov[j] = dOs[r * L::CS + 8 * jb + j];
                        dxv[j] = dXs[r * L::CS + 8 * jb + j];
                    }
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            acc[a][j] += qa[a] * dov[j] - ka[a] * dxv[j];
                }
                // every thread reads D only for its own block: write in place
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        Ds[(c0 + a) * L::SS + 8 * jb + j] = acc[a][j];
            }
        }
    }
    __syncthreads();
    if (dS0_out)
        for (int e = t; e < DK * kNV; e += kBT) {
            const int c = e / kNV, j = e % kNV;
            dS0_out[sbase + (long)c * DV + col0 + j] = Ds[c * L::SS + j];
        }
}

// out[i] = sum over slices s of part[s * n + i], s in order
__global__ __launch_bounds__(256) void sum_slices(const float *__restrict__ part, float *__restrict__ out, long n,
                                                  int nsl)
{
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        float s = part[i];
        for (int k2 = 1; k2 < nsl; ++k2)
            s += part[(long)k2 * n + i];
        out[i] = s;
    }
}

template <typename E, int DK>
hipError_t launch_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                      const float *S0, const void *dO, const float *dST, float *states, float *dq,
                      float *dk, float *dv, float *dg, float *dbeta, float *dS0, float *partials, int B,
                      int T, int H, int DV, hipStream_t stream)
{
    typedef BwdL<DK> L;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)bwd_kernel<E, DK>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    const int nbh = B * H, nsl = DV / kNV;
    const long rows = (long)B * T * H;
    float *pq = nsl > 1 ? partials : dq;
    float *pk = nsl > 1 ? partials + (long)nsl * rows * DK : dk;
    float *pg = nsl > 1 ? partials + 2L * nsl * rows * DK : dg;
    float *pb = nsl > 1 ? partials + 3L * nsl * rows * DK : dbeta;
    const int grid = ((nbh + kXCDs - 1) / kXCDs) * kXCDs * nsl;
    hipLaunchKernelGGL((bwd_kernel<E, DK>), dim3(grid), dim3(kBT), L::bytes, stream, (const E *)q,
                       (const E *)k, (const E *)v, (const E *)g, (const E *)beta, S0, (const E *)dO, dST,
                       states, dv, dS0, pq, pk, pg, pb, T, H, DV, nbh, nsl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsl == 1 || rows == 0)
        return e;
    const long nk = rows * DK;
    const int blocks = (int)((nk + 255) / 256 < 4096 ? (nk + 255) / 256 : 4096);
    hipLaunchKernelGGL(sum_slices, dim3(blocks), dim3(256), 0, stream, pq, dq, nk, nsl);
    hipLaunchKernelGGL(sum_slices, dim3(blocks), dim3(256), 0, stream, pk, dk, nk, nsl);
    hipLaunchKernelGGL(sum_slices, dim3(blocks), dim3(256), 0, stream, pg, dg, nk, nsl);
    const int bb = (int)((rows + 255) / 256 < 4096 ? (rows + 255) / 256 : 4096);
    hipLaunchKernelGGL(sum_slices, dim3(bb), dim3(256), 0, stream, pb, dbeta, rows, nsl);
    return hipGetLastError();
}

} // namespace

size_t chunk_bwd_workspace_floats(int B, int T, int H, int dk, int dv)
{
    const long nchunks = (T + kC - 1) / kC;
    const long nsl = dv / kNV;
    const long states = (nchunks > 1 ? nchunks - 1 : 0) * B * H * (long)dk * dv;
    const long parts = nsl > 1 ? nsl * (long)B * T * H * (3L * dk + 1) : 0;
    // each region rounded up to 64 floats (256 bytes)
    return (size_t)(((states + 63) / 64) * 64 + ((parts + 63) / 64) * 64);
}

hipError_t launch_chunk_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                            const float *S0, const void *dO, const float *dST, float *dq, float *dk,
                            float *dv, float *dg, float *dbeta, float *dS0, float *workspace, int B, int T,
                            int H, int DK, int DV, bool fp32, hipStream_t stream)
{
    const long nchunks = (T + kC - 1) / kC;
    const long sfl = (nchunks > 1 ? nchunks - 1 : 0) * B * H * (long)DK * DV;
    float *states = workspace;
    float *partials = workspace + ((sfl + 63) / 64) * 64;
    // 1. the incoming state of every chunk: the forward pass with a snapshot
    //    after every chunk (o not written)
    if (nchunks > 1) {
        Snapshots snap;
        snap.out = states;
        snap.every_chunks = 1;
        snap.count = (int)(nchunks - 1);
        hipError_t e = launch_chunk16(q, k, v, g, beta, S0, nullptr, nullptr, B, T, H, DK, DV, fp32, snap,
                                      stream);
        if (e != hipSuccess)
            return e;
    }
    // 2. the reverse walk (and the slice sums)
    if (fp32)
        return DK == 128 ? launch_bwd<float, 128>(q, k, v, g, beta, S0, dO, dST, states, dq, dk, dv, dg, dbeta,
                                                   dS0, partials, B, T, H, DV, stream)
                         : launch_bwd<float, 64>(q, k, v, g, beta, S0, dO, dST, states, dq, dk, dv, dg, dbeta,
                                                 dS0, partials, B, T, H, DV, stream);
    return DK == 128 ? launch_bwd<__bf16, 128>(q, k, v, g, beta, S0, dO, dST, states, dq, dk, dv, dg, dbeta,
                                                dS0, partials, B, T, H, DV, stream)
                     : launch_bwd<__bf16, 64>(q, k, v, g, beta, S0, dO, dST, states, dq, dk, dv, dg, dbeta,
                                              dS0, partials, B, T, H, DV, stream);
}

} // namespace kda
