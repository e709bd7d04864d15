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
// the range the pages' bound guarantees.  P is a running product of
// a_t = exp(g_t) (one exponential per element), Gam / P a running suffix
// product of the same a_t, and 1 / P = (Gam / P) * (1 / Gam) with one hardware
// reciprocal per channel and chunk (e^80 = 5.5e34 is far inside fp32).
//
// Work decomposition.  A workgroup owns one (sequence, head, 64-wide value
// slice); value columns of S never interact.  It runs 4 consumer wavefronts
// and NP producer wavefronts (8 in bf16 mode, 4 in fp32 test mode):
//   consumers 0..3  -- wavefront w keeps value columns [16w, 16w+16) of the
//                      dk x 64 fp32 state in MFMA accumulators for the whole
//                      sequence and runs the state-dependent products of every
//                      chunk in order; o goes straight to HBM;
//   producers       -- producer p owns chunks p, p+NP, p+2NP, ...: it loads q,
//                      k, g, v directly in its compute layout (lane = four key
//                      channels x eight tokens), builds the decayed operands in
//                      registers (prefix and suffix running products of exp(g);
//                      Kc = k / P from the suffix), and only then claims one of NS
//                      LDS slots, writes the consumers' operand images, issues
//                      the loads of its next chunk, forms A, M and the UT
//                      inverse on MFMA, and publishes the slot.
//                      Claiming the slot late keeps it held for the MFMA part
//                      only, so more chunks are in flight at once.
// Producers and consumers hand slots over through per-slot LDS flags ("ready"
// and per-consumer "done"); every wait is bounded and a WG-wide abort flag ends
// all waits if one ever runs out.  The kernel then still finishes, and it marks
// what it could not compute: the consumers write NaN in place of every o tile
// from the chunk at which they saw the abort on, and in place of the head
// slice's S_T (and any later snapshot).
//
// Instruction economy.  One wavefront issues at most one instruction every few
// cycles, so the consumer's per-chunk instruction count bounds the state chain:
// the slot holds -Kt so that X = V - Kt S accumulates straight onto V, O = Y +
// M U accumulates onto Y, the o tile and snapshot pointers advance by fixed
// steps, and every LDS operand read uses one base register plus an immediate.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_prep_unit.h"

namespace kda {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <typename E> struct Np { static constexpr int v = sizeof(E) == 2 ? 8 : 4; };
constexpr int kC = 16;                 // tokens per chunk
constexpr int kVS = 64;                // value columns per workgroup
constexpr int kXCDs = 8;
constexpr int kCUs = 256;
constexpr int kSpinLimit = 1 << 22;     // polls before a hand-off wait gives up
// s_waitcnt operand: vector-memory count 0, the other counters unconstrained
constexpr int kVmcntZero = 0x0F70;
// the same with at most 10 vector-memory operations outstanding (see kPubLag)
constexpr int kVmcntPub = 0x0F70 | 10;
// buffer-load cache policy of the gate workers' reads of what other CUs wrote:
// device scope, so the CU's own L1 never serves them
constexpr int kLoadDevice = 16;

// LDS layout.  Every MFMA operand is stored as the register image the reading
// wavefront loads (one contiguous 16- or 8-byte piece per lane), padded so that
// both the producer's writes and the consumers' reads are free of bank
// conflicts (64 banks of 4 bytes):
//   image16 (Kt, Qt, Kc): K-step m (32 channels), lane (l16 = token, g4):
//       element e of 8 at  m*MS + g4*GS + 8*l16 + e, GS = 136, MS = 4*GS; the
//       8 channels of (m, g4) are {32m + 4g4 + e} (e < 4) and {32m + 16 + 4g4 + e-4}
//       -- the contraction order the state accumulators impose (see consumer);
//   image4 (Ke^T, V^T): 16-row tile t, lane (l16 = channel or value, g4 =
//       token group): element e of 4 at  tile(t) + 4*(l16 + 16 g4) + e, with
//       tile(t) = t*KS + 8*((t/2) % 2), KS = 320 (the shift of every other tile
//       pair spreads the producer's 16-byte writes over all banks);
//   T, M: lane (l16 = row, g4): element e of 4 at 4*(l16 + 16 g4) + e = the
//       entry (row l16, column 4 g4 + e).
template <typename E, int DK>
struct WsL {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int NS = ES == 2 ? 6 : 3;        // LDS slots
    static constexpr int NP = Np<E>::v;               // producer wavefronts
    static constexpr int GS = 136, MS = 4 * GS;       // image16 strides (elements)
    static constexpr int KS = 320;                    // image4 tile stride (elements, >= 256 + 8)
    static constexpr int NKS = DK / 32, NCT = DK / 16;
    static constexpr int I16 = NKS * MS;              // elements of one image16
    // slot, E-typed part (element offsets)
    static constexpr int eKt = 0;                     // Kt image16
    static constexpr int eQt = eKt + I16;             // Qt image16
    static constexpr int eKe = eQt + I16;             // Ke^T image4, NCT tiles
    static constexpr int eV = eKe + NCT * KS;         // V^T image4, 4 tiles
    static constexpr int eT = eV + 4 * KS;            // T  [64 lanes][4]
    static constexpr int eM = eT + 256;               // M  [64 lanes][4]
    static constexpr int slotE = eM + 256;
    static constexpr int slotBytes = slotE * ES + DK * 4;   // + Gam fp32 [DK]
    static constexpr int pBytes = I16 * ES;           // producer scratch: Kc image16
    // byte offsets
    static constexpr int oSlots = 0;
    static constexpr int oProd = oSlots + NS * slotBytes;
    static constexpr int oFlags = oProd + NP * pBytes;
    static constexpr int nFlags = NS + NS * 4 + 1;    // ready[NS], done[NS][4], abort
    static constexpr int bytes = oFlags + nFlags * 4;
    static_assert(slotBytes % 32 == 0 && pBytes % 32 == 0, "alignment");
    static __device__ __forceinline__ int tile(int t) { return t * KS + 8 * ((t >> 1) & 1); }
    // image16 position of (token r, channel c)
    static __device__ __forceinline__ int img16(int r, int c)
    {
        const int m = c >> 5, cp = c & 31, hf = cp >> 4, cq = cp & 15;
        return m * MS + (cq >> 2) * GS + 8 * r + (cq & 3) + 4 * hf;
    }
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
// spin_limit polls the WG abort flag is raised and all later waits return.
// Returns whether the workgroup has aborted (read after the flags, so an abort
// raised before a flag was published is always seen).
__device__ __forceinline__ bool wait_flags(const int *f, int n, int stride, int target, int *abort_flag,
                                           int spin_limit)
{
    int spins = 0;
    for (;;) {
        bool ok = true;
        for (int i = 0; i < n; ++i)
            ok = ok && ld_flag(f + i * stride) >= target;
        if (ok || ld_flag(abort_flag))
            break;
        if (++spins > spin_limit) {
            st_flag(abort_flag, 1);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    const bool aborted = ld_flag(abort_flag) != 0;
    lds_fence();
    return aborted;
}

// A volatile LDS read (never fused with a neighbouring read into a wider one).
template <typename T>
__device__ __forceinline__ T lds_load(const unsigned char *p)
{
    return *(const volatile __attribute__((address_space(3))) T *)(p);
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
    // low halves of x and y (element 0 of each pair), high halves
    static __device__ __forceinline__ T los(T x, T y) { return (x & 0xffffu) | (y << 16); }
    static __device__ __forceinline__ T his(T x, T y) { return (x >> 16) | (y & 0xffff0000u); }
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int voff, int soff)
    {
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    }
};
template <> struct Pair<float> {
    typedef float2 T;
    static __device__ __forceinline__ float lo(T x) { return x.x; }
    static __device__ __forceinline__ float hi(T x) { return x.y; }
    static __device__ __forceinline__ T pack(float a, float b) { return make_float2(a, b); }
    static __device__ __forceinline__ T los(T x, T y) { return make_float2(x.x, y.x); }
    static __device__ __forceinline__ T his(T x, T y) { return make_float2(x.y, y.y); }
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int voff, int soff)
    {
        typedef unsigned v2u __attribute__((ext_vector_type(2)));
        const v2u x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        return make_float2(__uint_as_float(x[0]), __uint_as_float(x[1]));
    }
};

// Four adjacent elements as two packs: a = elements 0, 1, b = elements 2, 3.
template <typename E> struct Quad;
template <> struct Quad<__bf16> {
    unsigned a, b;
    static __device__ __forceinline__ Quad load(__amdgpu_buffer_rsrc_t r, int voff, int soff)
    {
        typedef unsigned v2u __attribute__((ext_vector_type(2)));
        const v2u x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        return Quad{x[0], x[1]};
    }
};
template <> struct Quad<float> {
    float2 a, b;
    static __device__ __forceinline__ Quad load(__amdgpu_buffer_rsrc_t r, int voff, int soff)
    {
        typedef unsigned v4u __attribute__((ext_vector_type(4)));
        const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
        return Quad{make_float2(__uint_as_float(x[0]), __uint_as_float(x[1])),
                    make_float2(__uint_as_float(x[2]), __uint_as_float(x[3]))};
    }
};

// A scalar element as raw bits (converted where it is used, so that no
// instruction right after the load has to wait for it).
__device__ __forceinline__ unsigned load_bits(__amdgpu_buffer_rsrc_t r, int voff, int soff, __bf16 *)
{
    return (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ unsigned load_bits(__amdgpu_buffer_rsrc_t r, int voff, int soff, float *)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ float bits_to_f(unsigned x, __bf16 *) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bits_to_f(unsigned x, float *) { return __uint_as_float(x); }
// A 16-token tile column of o: rows 4 g4 + j (j < 4) of this lane's column,
// row j at byte offset voff + j * stride.
__device__ __forceinline__ void store_o(__amdgpu_buffer_rsrc_t r, int voff, int stride, f32x4 x, __bf16 *)
{
    const unsigned lo = Pair<__bf16>::pack(x[0], x[1]), hi = Pair<__bf16>::pack(x[2], x[3]);
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)lo, r, voff, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(lo >> 16), r, voff, stride, 0);
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)hi, r, voff, 2 * stride, 0);
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(hi >> 16), r, voff, 3 * stride, 0);
}
__device__ __forceinline__ void store_o(__amdgpu_buffer_rsrc_t r, int voff, int stride, f32x4 x, float *)
{
#pragma unroll
    for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[j]), r, voff, j * stride, 0);
}

// Four packs (8 elements) stored contiguously.
__device__ __forceinline__ void st_quad(__bf16 *d, unsigned a, unsigned b, unsigned c, unsigned e)
{
    *reinterpret_cast<uint4 *>(d) = make_uint4(a, b, c, e);
}
__device__ __forceinline__ void st_quad(float *d, float2 a, float2 b, float2 c, float2 e)
{
    reinterpret_cast<float4 *>(d)[0] = make_float4(a.x, a.y, b.x, b.y);
    reinterpret_cast<float4 *>(d)[1] = make_float4(c.x, c.y, e.x, e.y);
}

// Two packs (4 elements) stored contiguously.
__device__ __forceinline__ void st_pair2(__bf16 *d, unsigned a, unsigned b)
{
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    *reinterpret_cast<v2u *>(d) = v2u{a, b};
}
__device__ __forceinline__ void st_pair2(float *d, float2 a, float2 b)
{
    *reinterpret_cast<float4 *>(d) = make_float4(a.x, a.y, b.x, b.y);
}

// Lane K of each 16-lane row of the wavefront, broadcast to the whole row
// (DPP row broadcast; folded into the consuming instruction).
template <int K>
__device__ __forceinline__ float row_bcast(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + K, 0xf, 0xf, false));
}

// S[16 ct + 4 g + j][.] *= Gam[16 ct + 4 g + j] for every ct < N, with lane
// 2 ct + j / 2 of row g holding Gam[16 ct + 4 g + j], j = 0..3, as gp.x (j even)
// and gp.y (j odd).
template <int N, int CT = 0>
__device__ __forceinline__ void decay_rows(f32x4 *S, f32x2 gp)
{
    if constexpr (CT < N) {
        S[CT][0] *= row_bcast<2 * CT>(gp.x);
        S[CT][1] *= row_bcast<2 * CT>(gp.y);
        S[CT][2] *= row_bcast<2 * CT + 1>(gp.x);
        S[CT][3] *= row_bcast<2 * CT + 1>(gp.y);
        decay_rows<N, CT + 1>(S, gp);
    }
}

// This lane's part of one head's dk x dv fp32 state from the accumulator
// strip: Sacc[ct][j] is S[16 ct + 4 g4 + j][col]; lane_off is the byte offset
// of S[4 g4][col].  One buffer over the head's state, uniform row offsets.
template <int NCT>
__device__ __forceinline__ void store_state(float *dst, const f32x4 (&Sacc)[NCT], int lane_off, int DV)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(dst, 0, NCT * 16 * DV * 4, 0x00020000);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Sacc[ct][j]), r, lane_off, (16 * ct + j) * DV * 4, 0);
}

// The same strip in the packed layout of the backward's workspace: element
// type E, element (r, c) at ((r / 4) DV + c) 4 + r % 4, so that the lane's four
// rows 16 ct + 4 g4 + j of one column are one contiguous piece; lane_off is the
// byte offset of the piece of (4 g4, col).  Lanes l16 of a row group g4 write
// 16 consecutive pieces (whole cache lines).
__device__ __forceinline__ void store_piece(__amdgpu_buffer_rsrc_t r, int voff, int soff, f32x4 x, __bf16 *)
{
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(v2u{Pair<__bf16>::pack(x[0], x[1]), Pair<__bf16>::pack(x[2], x[3])}, r,
                                          voff, soff, 0);
}
__device__ __forceinline__ void store_piece(__amdgpu_buffer_rsrc_t r, int voff, int soff, f32x4 x, float *)
{
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, x), r, voff, soff, 0);
}
template <typename E, int NCT>
__device__ __forceinline__ void store_state_packed(E *dst, const f32x4 (&Sacc)[NCT], int lane_off, int DV)
{
    constexpr int ES = (int)sizeof(E);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(dst, 0, NCT * 16 * DV * ES, 0x00020000);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
        store_piece(r, lane_off, ct * 4 * DV * 4 * ES, Sacc[ct], (E *)nullptr);
}

// Bytes spanned by `rows` rows of `width` bytes, `stride` bytes apart (0 rows: 0).
__device__ __forceinline__ int rows_bytes(int rows, int stride, int width)
{
    return rows > 0 ? (rows - 1) * stride + width : 0;
}

// Raw buffer over [base, base + bytes): loads past the end return 0 and stores
// past the end are dropped, which masks a chunk's ragged tail without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// One chunk's raw inputs in the producer's compute layout, straight from HBM
// (tokens past the end read 0).  Lane l = (cq, th) = (l % 32, l / 32) holds
// key channels 4cq .. 4cq+3 of g, k, q for tokens 8th .. 8th+7 (one 8-byte
// load per token and tensor); lane l = (vq, tq) = (l % 16, l / 16) holds value
// columns 4vq .. 4vq+3 of the slice for tokens 4tq .. 4tq+3; every lane holds
// beta of token l % 16 as raw bits (converted where used, so no instruction
// right after the loads waits).  29 loads: two chunks in flight stay within
// what the wave's outstanding-load counter tracks.  A chunk past the end is an
// empty buffer, so the loads are issued unconditionally (no branch for the
// wait-count analysis to merge conservatively).
template <typename E>
struct RawC {
    Quad<E> g[8], k[8], q[8], v[4];
    unsigned b;
};

template <typename E, int DK>
__device__ __forceinline__ void load_chunk(RawC<E> &R, const E *q, const E *k, const E *g, const E *v,
                                           const E *beta, long row0, int valid, int H, int DV, int slice,
                                           int lane)
{
    constexpr int ES = (int)sizeof(E);
    // row0 = (b T + t0) H + h: this head's row of the chunk's first token
    int rsk = H * DK * ES, rsv = H * DV * ES;
    // recompute the per-token scalar offsets at every call instead of keeping
    // them live across the whole loop (they would crowd out the SGPR file)
    asm volatile("" : "+s"(rsk), "+s"(rsv));
    const int nb = rows_bytes(valid, rsk, DK * ES);
    const __amdgpu_buffer_rsrc_t rq = buffer(q + row0 * DK, nb);
    const __amdgpu_buffer_rsrc_t rk = buffer(k + row0 * DK, nb);
    const __amdgpu_buffer_rsrc_t rg = buffer(g + row0 * DK, nb);
    const __amdgpu_buffer_rsrc_t rv = buffer(v + row0 * DV + slice * kVS, rows_bytes(valid, rsv, kVS * ES));
    const __amdgpu_buffer_rsrc_t rb = buffer(beta + row0, rows_bytes(valid, H * ES, ES));
    if (4 * (lane & 31) < DK) {
        const int vo = (lane & 31) * 4 * ES + (lane >> 5) * 8 * rsk;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            R.g[i] = Quad<E>::load(rg, vo, i * rsk);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            R.k[i] = Quad<E>::load(rk, vo, i * rsk);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            R.q[i] = Quad<E>::load(rq, vo, i * rsk);
    }
    const int vov = (lane & 15) * 4 * ES + (lane >> 4) * 4 * rsv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        R.v[i] = Quad<E>::load(rv, vov, i * rsv);
    R.b = load_bits(rb, (lane & 15) * H * ES, 0, (E *)nullptr);
}

// ---- the fused output gate (kda_chunk_fwd_gated) ------------------------------
// Page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section 3.2, output
// equation: y = Sigmoid(gate) * RMSNorm(o~) * w per (token, head), the norm over
// the head's dv readout columns -- which two value-slice workgroups produce.
// Consumer wavefront w of (head bh, slice) publishes in
// pub[(bh * nsl + slice) * 4 + w] how many of its chunks' o tiles have reached
// the L2, two chunks behind its stores (kPubLag).  Workgroups past the prefill
// grid are gate workers: each of their wavefronts takes (chunk, head) items of
// the heads whose workgroups run on its own XCD (the L2 that holds their tiles),
// in chunk order, waits until every consumer of the item's head has published
// the chunk, and overwrites the chunk's 16 rows of o with y in place.  The
// workers fill CUs the prefill grid leaves idle, and on each XCD they are
// dispatched after every prefill workgroup (workgroups start in index order),
// so the heads they wait for are already running and every wait ends; the
// waits are bounded all the same, and an item whose wait gives up is written
// as NaN (as is every later item of that wavefront).
constexpr int kPubLag = 2;

// One row piece of 8 elements (16 bytes in bf16, 32 in fp32).
template <typename E> struct Oct8;
template <> struct Oct8<__bf16> {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    u4 r;
    template <int AUX>
    static __device__ __forceinline__ Oct8 load(__amdgpu_buffer_rsrc_t rs, int voff)
    {
        return Oct8{(u4)__builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, AUX)};
    }
    __device__ __forceinline__ float get(int i) const
    {
        const unsigned x = r[i >> 1];
        return __uint_as_float((i & 1) ? (x & 0xffff0000u) : (x << 16));
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t rs, int voff, const float *v)
    {
        u4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[i] = Pair<__bf16>::pack(v[2 * i], v[2 * i + 1]);
        __builtin_amdgcn_raw_buffer_store_b128(x, rs, voff, 0, 0);
    }
};
template <> struct Oct8<float> {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    u4 a, b;
    template <int AUX>
    static __device__ __forceinline__ Oct8 load(__amdgpu_buffer_rsrc_t rs, int voff)
    {
        return Oct8{(u4)__builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, AUX),
                    (u4)__builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, 0, AUX)};
    }
    __device__ __forceinline__ float get(int i) const { return __uint_as_float(i < 4 ? a[i] : b[i - 4]); }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t rs, int voff, const float *v)
    {
        __builtin_amdgcn_raw_buffer_store_b128(u4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                                  __float_as_uint(v[3])},
                                               rs, voff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                                                  __float_as_uint(v[7])},
                                               rs, voff + 16, 0, 0);
    }
};

// Gate wavefront jw of the nw on XCD xcd.  Lane (sub, slot): LPU = DV / 8 lanes
// own one row, 8 contiguous elements each; a wavefront covers UPW rows at a
// time, NPASS passes per 16-row item.  The row's sum of squares is reduced over
// its LPU lanes with xor shuffles (which stay inside the row's aligned lane
// group).  Rows past T fall outside the item's buffers: their loads read 0 and
// their stores are dropped.  Software-pipelined by one item: the progress words
// and the gate rows of the next item are loaded before this item's y is stored.
template <typename E, int DV>
__device__ __forceinline__ void gate_worker(E *y, const E *gate, const float *w, float eps, const int *pub,
                                            int jw, int nw, int xcd, int nbh, int H, int T, int nsl,
                                            int spin_limit)
{
    constexpr int ES = (int)sizeof(E), LPU = DV / 8, UPW = 64 / LPU, NPASS = kC / UPW;
    const int lane = threadIdx.x & 63, sub = lane % LPU, slot = lane / LPU;
    const int nhx = nbh > xcd ? (nbh - xcd + kXCDs - 1) / kXCDs : 0;   // heads on this XCD
    const int nchunks = (T + kC - 1) / kC;
    const long items = (long)nhx * nchunks;
    if (jw >= items)
        return;
    float wv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        wv[i] = w ? w[8 * sub + i] : 1.f;
    const int nf = 4 * nsl;                                            // consumers per head
    const int rs = H * DV * ES;                                        // bytes between token rows
    const int lane_off = slot * rs + 8 * sub * ES;
    const float nanv = __builtin_nanf("");
    const int xcd_hw = hw_xcd();

    // item it: chunk c of head bh, buffers over its n <= 16 rows
    struct Item {
        int c, bh;
        __amdgpu_buffer_rsrc_t ry, rg, rp;
    };
    auto item = [&](long it) {
        Item m;
        m.c = (int)(it / nhx);
        m.bh = xcd + kXCDs * (int)(it % nhx);
        const int b = m.bh / H, h = m.bh % H, t0 = m.c * kC, n = T - t0 < kC ? T - t0 : kC;
        const long row0 = ((long)b * T + t0) * H + h;
        m.ry = buffer(y + row0 * DV, rows_bytes(n, rs, DV * ES));
        m.rg = buffer(gate + row0 * DV, rows_bytes(n, rs, DV * ES));
        m.rp = buffer(pub + (long)m.bh * nf, nf * 4);
        return m;
    };
    auto ld_pub = [&](const Item &m) {
        return (int)__builtin_amdgcn_raw_buffer_load_b32(m.rp, lane * 4, 0, kLoadDevice);
    };

    bool aborted = false;
    long it = jw;
    Item m = item(it);
    int f = ld_pub(m);
    Oct8<E> xg[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
        xg[p] = Oct8<E>::template load<2>(m.rg, lane_off + UPW * p * rs);     // read once: non-temporal
    for (;;) {
        // every consumer of the head has published chunk c (the first test, of the
        // words loaded one item ahead, sits outside the polling loop, so that it
        // waits only for those loads, not for everything issued since)
        if (!aborted && __builtin_amdgcn_ballot_w64(lane < nf && word_count(f) <= m.c) != 0) {
            int spins = 0;
            do {
                if (++spins > spin_limit) {
                    aborted = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
                f = ld_pub(m);
            } while (__builtin_amdgcn_ballot_w64(lane < nf && word_count(f) <= m.c) != 0);
        }
        // a consumer on another XCD: its tiles may sit in that XCD's L2
        if (__builtin_amdgcn_ballot_w64(lane < nf && word_xcd(f) != xcd_hw) != 0)
            aborted = true;
        Oct8<E> xo[NPASS];
#pragma unroll
        for (int p = 0; p < NPASS; ++p)
            xo[p] = Oct8<E>::template load<kLoadDevice>(m.ry, lane_off + UPW * p * rs);
        // the next item's progress words and gate rows
        const long nx = it + nw;
        const bool more = nx < items;
        Item mn = m;
        int fn = 0;
        Oct8<E> xgn[NPASS];
        if (more) {
            mn = item(nx);
            fn = ld_pub(mn);
#pragma unroll
            for (int p = 0; p < NPASS; ++p)
                xgn[p] = Oct8<E>::template load<2>(mn.rg, lane_off + UPW * p * rs);
        }
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            float x[8], ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] = xo[p].get(i);
                ss += x[i] * x[i];
            }
#pragma unroll
            for (int off = LPU / 2; off > 0; off >>= 1)
                ss += __shfl_xor(ss, off, 64);
            const float rr = gate_rms(ss, 1.0f / DV, eps);
            float yv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                yv[i] = aborted ? nanv : gate_elem(x[i], xg[p].get(i), rr, wv[i]);
            Oct8<E>::store(m.ry, lane_off + UPW * p * rs, yv);
        }
        if (!more)
            break;
        it = nx;
        m = mn;
        f = fn;
#pragma unroll
        for (int p = 0; p < NPASS; ++p)
            xg[p] = xgn[p];
    }
}

// ---- the fused preprocessing (kda_chunk_fwd_from_proj) --------------------------
// Page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section 3.2, input
// branches, and section 3.3, lower-bounded decay: the preprocessing of
// kda_prefill_prep (kda_prep_unit.h) runs in the prefill's own launch.  The first
// nprep workgroups are prep workers: in rounds, each group of four wavefronts
// maps one unit (two heads of this XCD over a 128-token tile), the round ends
// with every store acknowledged and a barrier, and then one tile flag per head
// goes out.  Units are dealt tile-major, so the workers sweep the sequence in
// step with the prefill, whose producers wait for the flag of a chunk's tile
// before loading the chunk (the flag is read one chunk ahead, so a set flag
// costs no wait).  The prep workers wait for nothing and are dispatched before
// every prefill workgroup, so the producers' waits end; they are bounded all
// the same (a give-up marks the workgroup's results NaN like any hand-off).
constexpr int kPrepKU = 16;            // tokens a prep lane loads ahead
constexpr int kMinPrepCUs = 96;        // fewest idle CUs the fused launch is used with

template <typename E> struct PrepArgs {
    const E *q_pre, *k_pre, *v_pre, *z, *beta_logit, *conv_init;
    const float *conv_w, *A;
    E *conv_final;
    int *done;          // [B*H][tiles]: 1 once the tile's outputs are in the L2
    int nprep;          // prep workgroups, a multiple of 8, numbered before the prefill's
};

template <typename E, int DK, int DV>
__device__ __forceinline__ void prep_worker(E *q, E *k, E *v, E *g, E *beta, const PrepArgs<E> &pa, int xcd,
                                            int r, int nwx, int nbh, int T, int H)
{
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int per = (int)blockDim.x / 256;                    // units per workgroup and round
    const int slot = wave >> 2, role = wave & 3;
    const int nhx = nbh > xcd ? (nbh - xcd + kXCDs - 1) / kXCDs : 0;   // heads on this XCD
    const int npx = (nhx + 1) / 2;                            // their pairs
    const int ntiles = (T + kTT - 1) / kTT;
    const long units = (long)npx * ntiles;
    const long nw = (long)nwx * per;
    for (long base = (long)r * per; base < units; base += nw) {
        const long u = base + slot;
        int bhA = 0, bhB = -1, tile = 0;
        if (u < units) {
            tile = (int)(u / npx);
            const int m = (int)(u % npx);
            bhA = xcd + kXCDs * (2 * m);
            bhB = 2 * m + 1 < nhx ? xcd + kXCDs * (2 * m + 1) : -1;
            prep_unit<E, DK, DV, kPrepKU>(pa.q_pre, pa.k_pre, pa.v_pre, pa.conv_w, pa.conv_init, pa.z, pa.A,
                                          pa.beta_logit, q, k, v, g, beta, pa.conv_final, T, H, bhA, bhB, tile,
                                          role, lane);
        }
        // every store of the round acknowledged (in the L2), then the flags
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __syncthreads();
        if (role == 0 && u < units) {
            const int word = tag_xcd(1, hw_xcd());
            __builtin_amdgcn_raw_buffer_store_b32(word, buffer(pa.done + (long)bhA * ntiles + tile, 4), 4 * lane, 0,
                                                  0);
            if (bhB >= 0)
                __builtin_amdgcn_raw_buffer_store_b32(word, buffer(pa.done + (long)bhB * ntiles + tile, 4), 4 * lane,
                                                      0, 0);
        }
    }
}

// MODE 0: the plain prefill.  MODE 1 (GATED): the fused output gate -- o is y's
// buffer (the consumers' tiles, gated in place by the workers), the consumers
// publish their progress in pub, and the workgroups from grid_p on are gate
// workers (ngate of them, a multiple of 8).  MODE 2 (PROJ): the fused
// preprocessing -- the first pa.nprep workgroups are prep workers writing q, k,
// v, g, beta, which the prefill workgroups after them read.
template <typename E, int DK, int MODE>
__global__ __launch_bounds__(64 * (4 + Np<E>::v)) void prefill_ws_kernel(
    const E *q, const E *k, const E *v, const E *g, const E *beta, const float *S0, E *o,
    float *S_T, float *snaps, int snap_chunks, int n_snaps, int snap_packed, int T, int H, int DV, int nbh,
    int nsl, int spin_limit, int *pub, const E *gate, const float *gate_w, float gate_eps, int grid_p,
    int ngate, PrepArgs<E> pa)
{
    constexpr bool GATED = MODE == 1, PROJ = MODE == 2;
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
    int id = blockIdx.x;
    if constexpr (PROJ) {
        if (id < pa.nprep) {
            // nprep is a multiple of 8: prep worker id shares the XCD of every id' = id mod 8
            if (DV == 128)
                prep_worker<E, DK, 128>(const_cast<E *>(q), const_cast<E *>(k), const_cast<E *>(v),
                                        const_cast<E *>(g), const_cast<E *>(beta), pa, id % kXCDs, id / kXCDs,
                                        pa.nprep / kXCDs, nbh, T, H);
            else
                prep_worker<E, DK, 64>(const_cast<E *>(q), const_cast<E *>(k), const_cast<E *>(v),
                                       const_cast<E *>(g), const_cast<E *>(beta), pa, id % kXCDs, id / kXCDs,
                                       pa.nprep / kXCDs, nbh, T, H);
            return;
        }
        id -= pa.nprep;
    }
    const int xcd = id % kXCDs, rr = id / kXCDs;
    if constexpr (GATED) {
        if (id >= grid_p) {
            // grid_p is a multiple of 8: worker j = id - grid_p shares the XCD of every id' = j mod 8
            const int waves = 4 + L::NP, j = id - grid_p;
            const int jw = (j / kXCDs) * waves + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
            const int nw = (ngate / kXCDs) * waves;
            if (DV == 128)
                gate_worker<E, 128>(o, gate, gate_w, gate_eps, pub, jw, nw, xcd, nbh, H, T, nsl, spin_limit);
            else
                gate_worker<E, 64>(o, gate, gate_w, gate_eps, pub, jw, nw, xcd, nbh, H, T, nsl, spin_limit);
            return;
        }
    }
    const int bh = (rr / nsl) * kXCDs + xcd, slice = rr % nsl;
    if (bh >= nbh)
        return;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    // wavefront index, made provably uniform (buffer descriptors built from it
    // must live in scalar registers)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const long tokb = (long)b * T;
    const int nchunks = (T + kC - 1) / kC;

    for (int i = tid; i < L::nFlags; i += 64 * (4 + L::NP))
        flags[i] = 0;
    __syncthreads();

    if (wave < 4) {
        // =============================== consumer ===============================
        // the state chain is the critical path: let it win issue slots
        __builtin_amdgcn_s_setprio(2);
        const int w = wave;
        const int col = slice * kVS + 16 * w + l16;      // this lane's value column
        f32x4 Sacc[NCT];                                  // S[16 ct + 4 g4 + j][col]
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Sacc[ct][j] = S0 ? S0[((long)bh * DK + 16 * ct + 4 * g4 + j) * DV + col] : 0.f;
        // drain the initial-state loads here: left pending into the loop, they
        // make every chunk wait for all of its outstanding memory operations
        // (the o stores included) before the state can be touched
        __builtin_amdgcn_s_waitcnt(kVmcntZero);

        // o: this wave's 16 x 16 tile of chunk c; lane (l16 = column, g4) writes
        // rows 4 g4 .. 4 g4 + 3.  The tile base advances by a fixed step per
        // chunk; only the last chunk can be ragged (rows past T fall outside the
        // buffer and are dropped).
        const int rso = H * DV * L::ES;                   // bytes between token rows of o
        const int ovo = (4 * g4) * rso + l16 * L::ES;
        long ooff = (tokb * H + h) * (long)DV + slice * kVS + 16 * w;   // o tile of chunk 0
        const long ostep = (long)kC * H * DV;
        // o == nullptr (an internal caller that only wants states): every store
        // falls outside an empty buffer and is dropped
        const int ofull = o ? rows_bytes(kC, rso, 16 * L::ES) : 0;
        const int olast = o ? rows_bytes(T - (nchunks - 1) * kC, rso, 16 * L::ES) : 0;
        // gated: this wavefront's progress word (lane 0 writes it; the other
        // lanes' offsets fall outside the 4-byte buffer)
        __amdgpu_buffer_rsrc_t rpub;
        int xcd_hw = 0;
        if constexpr (GATED) {
            rpub = buffer(pub + ((long)bh * nsl + slice) * 4 + w, 4);
            xcd_hw = hw_xcd();
        }

        // this lane's byte offsets inside a slot: image16 pieces (Kt, Qt),
        // image4 pieces (Ke^T, V^T, T, M) and the Gam pair (see decay_rows)
        const int laA = (g4 * L::GS + 8 * l16) * L::ES;
        const int laB = 4 * lane * L::ES;
        const int laC = L::slotE * L::ES + (16 * (l16 >> 1) + 4 * g4 + 2 * (l16 & 1)) * 4;

        // Chunk c's operands, read from its slot into registers one chunk ahead:
        // the state chain of chunk c then runs with no LDS wait in it, while the
        // reads for chunk c + 1 overlap chunk c's state update.  The reads are
        // volatile so that none is fused with a neighbour into a wider read whose
        // halves would then have to be copied into the operand tuples.
        // The A operands of the 16-deep products (T, M, Ke^T) sit in the low half
        // of 8-element tuples whose high half stays zero for the whole loop (the
        // zero is opaque to the compiler, so it is never rematerialised).
        struct Ops {
            V8 kt[NKS], qt[NKS];
            V8 tr, mr, kr[NCT];
            V4 vv;
            f32x2 gp;         // Gam pair, see decay_rows
        };
        auto low = [](V4 x, V8 keep) { return __builtin_shufflevector(cat8(x, x), keep, 0, 1, 2, 3, 12, 13, 14, 15); };
        auto rd8 = [&](int s, int off) { return lds_load<V8>(smem + L::oSlots + s * L::slotBytes + off); };
        auto rd4 = [&](int s, int off) { return lds_load<V4>(smem + L::oSlots + s * L::slotBytes + off); };
        auto fetch = [&](Ops &op, int s, int c) {
            const bool ab = wait_flags(ready + s, 1, 1, c + 1, abort_flag, spin_limit);
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                op.kt[m] = rd8(s, laA + (L::eKt + m * L::MS) * L::ES);
                op.qt[m] = rd8(s, laA + (L::eQt + m * L::MS) * L::ES);
            }
            op.vv = rd4(s, laB + (L::eV + L::tile(w)) * L::ES);
            op.tr = low(rd4(s, laB + L::eT * L::ES), op.tr);
            op.mr = low(rd4(s, laB + L::eM * L::ES), op.mr);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                op.kr[ct] = low(rd4(s, laB + (L::eKe + L::tile(ct)) * L::ES), op.kr[ct]);
            op.gp = lds_load<f32x2>(smem + L::oSlots + s * L::slotBytes + laC);
            return ab;
        };

        Ops op;
        V8 bxv, buv;            // B operands of the 16-deep products, high half zero
        {
            V8 z = {};
            asm volatile("" : "+v"(z));
            op.tr = op.mr = bxv = buv = z;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                op.kr[ct] = z;
        }
        const int lane_soff = ((4 * g4) * DV + col) * 4;   // byte offset of S[4 g4][col] in a state
        // snapshots: fp32 row-major, or the packed layout (lane piece (g4, col))
        const int snap_es = snap_packed ? L::ES : 4;
        const int lane_poff = (g4 * DV + col) * 4 * L::ES;
        int snap_left = snap_chunks, snap_idx = 0;
        char *snap_dst = snaps ? reinterpret_cast<char *>(snaps) + (long)bh * DK * DV * snap_es : nullptr;
        const long snap_step = (long)nbh * DK * DV * snap_es;
        // the packed workspace starts with the initial state
        if (snap_dst && snap_packed) {
            store_state_packed(reinterpret_cast<E *>(snap_dst), Sacc, lane_poff, DV);
            snap_dst += snap_step;
        }
        int s = 0;                                        // slot of chunk c
        // set once a hand-off wait of this workgroup gave up: from then on the
        // results are marked (NaN) instead of written
        bool aborted = false;
        const f32x4 nan4 = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        if (nchunks > 0)
            aborted = fetch(op, 0, 0);
        for (int c = 0; c < nchunks; ++c) {
            // S strip as B operands; contraction slice m holds channels
            // {32m + 4 g4 + e, 32m + 16 + 4 g4 + e}, e = 0..3
            V8 Bs[NKS];
#pragma unroll
            for (int m = 0; m < NKS; ++m)
                Bs[m] = cat8(cvt4<E>(Sacc[2 * m]), cvt4<E>(Sacc[2 * m + 1]));
            // X = V - Kt S: the slot holds -Kt, so the accumulator starts at V
            // (rows 4 g4 + j = tokens, column l16); Y = Qt S
            f32x4 X, Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                X[j] = to_f(op.vv[j]);
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                X = mma32(op.kt[m], Bs[m], X);
                Y = mma32(op.qt[m], Bs[m], Y);
            }
            // U = T X, then O = Y + M U   (contraction over tokens 4 g4 + e; the
            // zero high halves of A and B cancel)
            bxv = low(cvt4<E>(X), bxv);
            const f32x4 U = mma32(op.tr, bxv, f32x4{0.f, 0.f, 0.f, 0.f});
            buv = low(cvt4<E>(U), buv);
            const f32x4 O = mma32(op.mr, buv, Y);
            // S <- Gam S + Ke^T U
            decay_rows<NCT>(Sacc, op.gp);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                Sacc[ct] = mma32(op.kr[ct], buv, Sacc[ct]);
            // the state after chunk c, when c + 1 closes a snapshot block
            if (snaps) {
                if (--snap_left == 0) {
                    snap_left = snap_chunks;
                    if (snap_idx < n_snaps) {
                        f32x4 Sout[NCT];
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct)
                            Sout[ct] = aborted ? nan4 : Sacc[ct];
                        if (snap_packed)
                            store_state_packed(reinterpret_cast<E *>(snap_dst), Sout, lane_poff, DV);
                        else
                            store_state(reinterpret_cast<float *>(snap_dst), Sout, lane_soff, DV);
                    }
                    ++snap_idx;
                    snap_dst += snap_step;
                }
            }
            // every read of slot s is in registers (and consumed): hand it back,
            // then fetch the next chunk while the state update runs
            lds_fence();
            st_flag(done + s * 4 + w, c + 1);
            s = s + 1 == NS ? 0 : s + 1;
            if (c + 1 < nchunks)
                aborted |= fetch(op, s, c + 1);
            else
                aborted |= ld_flag(abort_flag) != 0;
            const __amdgpu_buffer_rsrc_t ro = buffer(o ? o + ooff : o, c + 1 < nchunks ? ofull : olast);
            store_o(ro, ovo, rso, aborted ? nan4 : O, (E *)nullptr);
            ooff += ostep;
            if constexpr (GATED) {
                // Per chunk this wavefront issues 4 o stores and this 1 progress
                // store (and no other vector-memory operation: the gated entry
                // writes no snapshots), so once at most 10 are outstanding the
                // o tiles of chunk c - 2 and all before it are in the L2.
                __builtin_amdgcn_s_waitcnt(kVmcntPub);
                __builtin_amdgcn_raw_buffer_store_b32(tag_xcd(c + 1 - kPubLag > 0 ? c + 1 - kPubLag : 0, xcd_hw), rpub,
                                                      4 * lane, 0, 0);
            }
        }
        if constexpr (GATED) {
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            __builtin_amdgcn_raw_buffer_store_b32(tag_xcd(nchunks, xcd_hw), rpub, 4 * lane, 0, 0);
        }
        if (S_T) {
            aborted |= ld_flag(abort_flag) != 0;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                Sacc[ct] = aborted ? nan4 : Sacc[ct];
            store_state(S_T + (long)bh * DK * DV, Sacc, lane_soff, DV);
        }
        return;
    }

    // ================================= producer =================================
    const int pw = wave - 4;
    E *pKc = reinterpret_cast<E *>(smem + L::oProd + pw * L::pBytes);
    const long hrow = (long)b * T * H + h;       // row of token 0 of this head

    auto load_raw = [&](RawC<E> &R, int c) {
        const int t0 = c * kC;
        load_chunk<E, DK>(R, q, k, g, v, beta, hrow + (long)t0 * H, T - t0 < kC ? T - t0 : kC, H, DV, slice, lane);
    };
    // PROJ: a chunk is loaded once its tile's flag is set.  ptile holds the flag of
    // the chunk this producer loads next, read together with the previous chunk.
    const int ntiles = (T + kTT - 1) / kTT;
    int ptile = 1;
    auto tile_flag = [&](int c) {
        return (int)__builtin_amdgcn_raw_buffer_load_b32(buffer(pa.done + (long)bh * ntiles, ntiles * 4),
                                                         ((c * kC) / kTT) * 4, 0, kLoadDevice);
    };
    const int xcd_hw = PROJ ? hw_xcd() : 0;
    auto load = [&](RawC<E> &R, int c) {
        if constexpr (PROJ) {
            if (c < nchunks) {
                if (ptile == 0) {
                    int spins = 0;
                    while ((ptile = tile_flag(c)) == 0) {
                        if (ld_flag(abort_flag))
                            break;
                        if (++spins > spin_limit) {
                            st_flag(abort_flag, 1);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                }
                // written on another XCD: the tile may sit in that XCD's L2
                if (ptile != 0 && word_xcd(ptile) != xcd_hw)
                    st_flag(abort_flag, 1);
            }
            ptile = c + L::NP < nchunks ? tile_flag(c + L::NP) : tag_xcd(1, xcd_hw);
        }
        load_raw(R, c);
    };

    // One chunk from raw registers to a published slot.
    auto produce = [&](RawC<E> &raw, int c) {
        typedef typename PE::T PT;
        const int s = c % NS;
        // lane coordinates re-derived per chunk: the masks and selects built from
        // them below are cheap, and hoisting them all out of the loop would not
        // fit the register files
        int r16 = l16, rg4 = g4;
        asm volatile("" : "+v"(r16), "+v"(rg4));

        // The operands are built in registers first and written to the slot only
        // once it is free: a slot is then held for the MFMA part of the chunk
        // alone, not for its elementwise part too, so more chunks are in flight.
        // ---- V^T pieces: lane (vq, tq) holds value columns 4vq .. 4vq+3 for token
        // group tq (two 8-element pieces: columns 4vq, +1 and 4vq+2, +3) --------
        PT vtp[8];
        vtp[0] = PE::los(raw.v[0].a, raw.v[1].a), vtp[1] = PE::los(raw.v[2].a, raw.v[3].a);
        vtp[2] = PE::his(raw.v[0].a, raw.v[1].a), vtp[3] = PE::his(raw.v[2].a, raw.v[3].a);
        vtp[4] = PE::los(raw.v[0].b, raw.v[1].b), vtp[5] = PE::los(raw.v[2].b, raw.v[3].b);
        vtp[6] = PE::his(raw.v[0].b, raw.v[1].b), vtp[7] = PE::his(raw.v[2].b, raw.v[3].b);

        // ---- decay factors by running products, then the operands ------------
        // Lane (cq, th): key channels 4cq + u (u < 4), tokens 8th + i (i < 8).
        // The two halves of the chunk meet through the partner lane l ^ 32.
        const bool ew = 4 * (lane & 31) < DK;
        const int cq = lane & 31, th = lane >> 5;
        const int io = L::img16(8 * th, 4 * cq);          // token 8th + i adds 8 i
        PT ktp[8][2], qtp[8][2], kep[2][8];
        float gm4[4];
        if (ew) {
            float al[4][8];                               // alpha = e^g
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                al[0][i] = __builtin_amdgcn_exp2f(PE::lo(raw.g[i].a) * 1.4426950408889634f);
                al[1][i] = __builtin_amdgcn_exp2f(PE::hi(raw.g[i].a) * 1.4426950408889634f);
                al[2][i] = __builtin_amdgcn_exp2f(PE::lo(raw.g[i].b) * 1.4426950408889634f);
                al[3][i] = __builtin_amdgcn_exp2f(PE::hi(raw.g[i].b) * 1.4426950408889634f);
            }
            // each half's total (a product tree over its 8 tokens); the partner's
            // total starts the second half's prefix and completes Gam = e^{G_15}
            float oth[4], sf[4], ig[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float t01 = al[u][0] * al[u][1], t23 = al[u][2] * al[u][3];
                const float t45 = al[u][4] * al[u][5], t67 = al[u][6] * al[u][7];
                const float tot = (t01 * t23) * (t45 * t67);
                oth[u] = __shfl_xor(tot, 32, 64);
                gm4[u] = tot * oth[u];
                sf[u] = th ? 1.f : oth[u];
                ig[u] = __builtin_amdgcn_rcpf(gm4[u]);    // 1 / Gam: one reciprocal per channel
            }
            // running suffix Gam / P_r = prod_{s > r} alpha_s (no division per
            // element); Ke = k Gam / P, Kc = k / P = Ke (1 / Gam).  Gam >= e^-80 is
            // a normal float, so 1 / Gam <= e^80 is finite.
            // kep[i / 4][2u + (i % 4) / 2] packs channel u of tokens i, i + 1 (i even)
            float es[4];
#pragma unroll
            for (int i = 7; i >= 0; --i) {
                float kk[4], kc[4];
                kk[0] = PE::lo(raw.k[i].a), kk[1] = PE::hi(raw.k[i].a), kk[2] = PE::lo(raw.k[i].b), kk[3] = PE::hi(raw.k[i].b);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float e = kk[u] * sf[u];
                    kc[u] = e * ig[u];
                    if (i & 1)
                        es[u] = e;
                    else
                        kep[i >> 2][2 * u + ((i & 3) >> 1)] = PE::pack(e, es[u]);
                    if (i > 0)
                        sf[u] *= al[u][i];
                }
                // Kc only feeds this producer's own products: its private image
                st_pair2(pKc + io + 8 * i, PE::pack(kc[0], kc[1]), PE::pack(kc[2], kc[3]));
            }
            // running prefix P_r = e^{G_r}; Kt = k P, Qt = q P
            float p[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                p[u] = th ? oth[u] : 1.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float kk[4], qq[4];
                kk[0] = PE::lo(raw.k[i].a), kk[1] = PE::hi(raw.k[i].a), kk[2] = PE::lo(raw.k[i].b), kk[3] = PE::hi(raw.k[i].b);
                qq[0] = PE::lo(raw.q[i].a), qq[1] = PE::hi(raw.q[i].a), qq[2] = PE::lo(raw.q[i].b), qq[3] = PE::hi(raw.q[i].b);
                float kt[4], qt[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    p[u] *= al[u][i];
                    kt[u] = -(kk[u] * p[u]);   // stored negated (see the consumer)
                    qt[u] = qq[u] * p[u];
                }
                ktp[i][0] = PE::pack(kt[0], kt[1]), ktp[i][1] = PE::pack(kt[2], kt[3]);
                qtp[i][0] = PE::pack(qt[0], qt[1]), qtp[i][1] = PE::pack(qt[2], qt[3]);
            }
        }
        const unsigned braw = raw.b;

        // ---- claim the slot, then write the consumers' operand images ----------
        if (c >= NS)
            wait_flags(done + s * 4, 4, 1, c - NS + 1, abort_flag, spin_limit);
        // while it holds the slot the producer issues ahead of the other producer
        // on its SIMD (still behind the consumer): the time a slot is held bounds
        // how many chunks are in flight
        __builtin_amdgcn_s_setprio(1);
        E *sl = reinterpret_cast<E *>(smem + L::oSlots + s * L::slotBytes);
        float *gam = reinterpret_cast<float *>(smem + L::oSlots + s * L::slotBytes + L::slotE * L::ES);
        {
            const int vq = lane & 15, tq = lane >> 4;
            E *vt = sl + L::eV + L::tile(vq >> 2) + 4 * (4 * (vq & 3) + 16 * tq);
            st_quad(vt, vtp[0], vtp[1], vtp[2], vtp[3]);
            st_quad(vt + 8, vtp[4], vtp[5], vtp[6], vtp[7]);
        }
        if (ew) {
            if (th == 0)
                *reinterpret_cast<f32x4 *>(gam + 4 * cq) = f32x4{gm4[0], gm4[1], gm4[2], gm4[3]};
            E *ke = sl + L::eKe + L::tile(cq >> 2) + 4 * (4 * (cq & 3) + 32 * th);   // token group 2th + j adds 64 j
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                st_pair2(sl + L::eKt + io + 8 * i, ktp[i][0], ktp[i][1]);
                st_pair2(sl + L::eQt + io + 8 * i, qtp[i][0], qtp[i][1]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                st_quad(ke + 64 * j, kep[j][0], kep[j][1], kep[j][2], kep[j][3]);
                st_quad(ke + 64 * j + 8, kep[j][4], kep[j][5], kep[j][6], kep[j][7]);
            }
        }
        // the next chunk's loads, once this chunk's raw registers are dead
        load(raw, c + L::NP);
        lds_fence();

        // ---- A and M on MFMA (contraction over the DK channels) ----------------
        f32x4 Ar = {0.f, 0.f, 0.f, 0.f}, ATr = {0.f, 0.f, 0.f, 0.f}, Mtr = {0.f, 0.f, 0.f, 0.f};
        {
            const int ia = g4 * L::GS + 8 * l16;
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                const V8 ak = *reinterpret_cast<const V8 *>(sl + L::eKt + ia + m * L::MS);
                const V8 aq = *reinterpret_cast<const V8 *>(sl + L::eQt + ia + m * L::MS);
                const V8 bc = *reinterpret_cast<const V8 *>(pKc + ia + m * L::MS);
                Ar = mma32(ak, bc, Ar);         // <Kt_r, Kc_i>: rows r = 4 g4 + j, column i = l16
                ATr = mma32(bc, ak, ATr);       // <Kc_i, Kt_r>: rows i = 4 g4 + j, column r = l16
                Mtr = mma32(bc, aq, Mtr);       // <Kc_i, Qt_r>: rows i = 4 g4 + j, column r = l16
            }
            // M^T's accumulator is already M's image: entry (row l16, column 4 g4 + j),
            // kept where column <= row
            f32x4 Mm;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Mm[j] = 4 * rg4 + j <= r16 ? Mtr[j] : 0.f;
            *reinterpret_cast<V4 *>(sl + L::eM + 4 * lane) = cvt4<E>(Mm);
        }

        // ---- T = (I + A)^{-1} Diag(beta), A[r][i] = beta_r <Kt_r, Kc_i> (i < r) ----
        // A is strictly lower triangular, so A^16 = 0 and, exactly,
        //   (I + A)^{-1} = sum_k (-A)^k = (I - A)(I + A^2)(I + A^4)(I + A^8).
        // Evaluated on MFMA with every 16 x 16 matrix in the accumulator layout
        // (lane (n, g) holds rows 4g .. 4g+3 of column n).  mul(Xt, Y) forms X Y
        // from X^T and Y in that layout: lane (n, g)'s four elements are the
        // contraction indices 4g .. 4g+3 of both operands; so (XY)^T = mul(Y, X^T)
        // comes from the same registers.  Each product is one 16-deep MFMA in
        // the element type: the operands are rounded to bf16 in bf16 mode (the
        // result is rounded to bf16 for the consumers anyway, and the powers of
        // A only refine it), accumulation is fp32.  The consumers take
        // T as an MFMA A operand, whose image is T^T in the accumulator layout:
        //   T^T = Diag(beta) (I - A^T)(I + A2^T)(I + A4^T)(I + A8^T),
        // built from A and A^T (both straight from the bf16 products above).
        {
            auto mul = [](f32x4 xt, f32x4 y) {
                return mma16(cvt4<E>(xt), cvt4<E>(y), f32x4{0.f, 0.f, 0.f, 0.f});
            };
            // beta of token l16 (row l16 of A^T's columns) and of tokens 4g + j
            // (this lane's rows), the latter fetched from lanes 4g + j
            const float bl = bits_to_f(braw, (E *)nullptr);
            f32x4 br;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                br[j] = bits_to_f((unsigned)__builtin_amdgcn_ds_bpermute(4 * (4 * rg4 + j), (int)braw), (E *)nullptr);
            f32x4 I4, A, AT;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 4 * rg4 + j;
                I4[j] = row == r16 ? 1.f : 0.f;
                A[j] = row > r16 ? -br[j] * Ar[j] : 0.f;     // A[row][l16] (Ar holds -<Kt, Kc>)
                AT[j] = row < r16 ? -bl * ATr[j] : 0.f;      // A^T[row][l16] = A[l16][row]
            }
            if constexpr (sizeof(E) == 2) {
                const f32x4 A2 = mul(AT, A), A2T = mul(A, AT);
                const f32x4 A4 = mul(A2T, A2), A4T = mul(A2, A2T);
                const f32x4 A8T = mul(A4, A4T);
                const f32x4 WT = I4 + A4T + A8T + mul(A4, A8T);   // ((I + A^4)(I + A^8))^T
                const f32x4 W2T = WT + mul(A2, WT);                // (I + A2^T) W^T
                const f32x4 LiT = W2T - mul(A, W2T);               // (I - A^T) W2^T = ((I + A)^{-1})^T
                *reinterpret_cast<V4 *>(sl + L::eT + 4 * lane) = cvt4<E>(br * LiT);
            } else {
                // fp32 test mode: forward substitution.  The product form loses
                // about the size of its intermediate powers in accuracy (C(14, 7) =
                // 3432 for A all ones below the diagonal: identical keys, beta = 1,
                // no decay), which fp32 results must not; lane i < 16 solves column
                // i of (I + A) L = I from A staged in this producer's Kc scratch (its
                // reads by the MFMAs above have completed).
                float *As = reinterpret_cast<float *>(pKc);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    As[(4 * rg4 + j) * 17 + r16] = A[j];
                if (lane < kC) {
                    float x[kC];
#pragma unroll
                    for (int r = 0; r < kC; ++r) {
                        float acc = r == lane ? 1.f : 0.f;
#pragma unroll
                        for (int j = 0; j < r; ++j)
                            acc -= As[r * 17 + j] * x[j];
                        x[r] = acc;
                        // T[r][lane] = L[r][lane] beta_lane at (row r, column lane) of the image
                        sl[L::eT + 4 * (r + 16 * (lane >> 2)) + (lane & 3)] = (E)(acc * bl);
                    }
                }
            }
        }
        // publish the slot
        lds_fence();
        if (lane == 0)
            st_flag(ready + s, c + 1);
        __builtin_amdgcn_s_setprio(0);
    };

    // one chunk in flight per producer: the loads for chunk c + NP are issued
    // as soon as chunk c's raw registers have been consumed
    RawC<E> raw;
    if constexpr (PROJ)
        ptile = pw < nchunks ? tile_flag(pw) : tag_xcd(1, xcd_hw);
    load(raw, pw);
    for (int c = pw; c < nchunks; c += L::NP)
        produce(raw, c);
}

// pub[i] = 0 for i < n (the consumers' progress words of one gated call)
__global__ __launch_bounds__(256) void zero_pub(int *pub, long n)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        pub[i] = 0;
}

// What a launch fuses into the prefill: nothing (MODE 0), the output gate (og,
// with o = y's buffer and pub the caller's nbh * nsl * 4 progress words; MODE 1)
// or the preprocessing (prep, with q, k, v, g, beta its outputs and done the
// caller's nbh * tiles flags; MODE 2).
struct Fusion {
    const OutputGate *og = nullptr;
    int *pub = nullptr;
    const PrepInputs *prep = nullptr;
    int *done = nullptr;
};

template <typename E, int DK, int MODE>
hipError_t launch_ws(const void *q, const void *k, const void *v, const void *g, const void *beta,
                     const float *S0, void *o, float *S_T, int B, int T, int H, int dv,
                     const Snapshots &snap, int spin_limit, const Fusion &fu, hipStream_t stream)
{
    typedef WsL<E, DK> L;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    // above half the LDS: one workgroup per CU, so a gate or prep worker never
    // shares a CU with a prefill workgroup
    constexpr int lds = L::bytes > 81 * 1024 ? L::bytes : 81 * 1024;
    // a per-device function attribute: set on every call (cheap, and correct
    // whichever device and thread the call comes from)
    hipError_t e = hipFuncSetAttribute((const void *)prefill_ws_kernel<E, DK, MODE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess)
        return e;
    const int nbh = B * H, nsl = dv / kVS;
    const int grid_p = ((nbh + kXCDs - 1) / kXCDs) * kXCDs * nsl;
    int ngate = 0;
    PrepArgs<E> pa = {};
    if constexpr (MODE == 1) {
        // the CUs the prefill grid leaves idle, at least 8 per XCD (which start as
        // prefill workgroups finish when the grid fills the chip)
        ngate = kCUs - grid_p > 64 ? ((kCUs - grid_p) / kXCDs) * kXCDs : 64;
        const long npub = (long)nbh * nsl * 4;
        hipLaunchKernelGGL(zero_pub, dim3((unsigned)((npub + 255) / 256)), dim3(256), 0, stream, fu.pub, npub);
    }
    if constexpr (MODE == 2) {
        // the CUs the prefill grid leaves idle (at least kMinPrepCUs)
        const PrepInputs &pi = *fu.prep;
        pa.q_pre = (const E *)pi.q_pre;
        pa.k_pre = (const E *)pi.k_pre;
        pa.v_pre = (const E *)pi.v_pre;
        pa.z = (const E *)pi.z;
        pa.beta_logit = (const E *)pi.beta_logit;
        pa.conv_init = (const E *)pi.conv_init;
        pa.conv_w = pi.conv_w;
        pa.A = pi.A;
        pa.conv_final = (E *)pi.conv_final;
        pa.done = fu.done;
        pa.nprep = ((kCUs - grid_p) / kXCDs) * kXCDs;
        const long ndone = (long)nbh * ((T + kTT - 1) / kTT);
        hipLaunchKernelGGL(zero_pub, dim3((unsigned)((ndone + 255) / 256)), dim3(256), 0, stream, fu.done, ndone);
    }
    const OutputGate *og = fu.og;
    hipLaunchKernelGGL((prefill_ws_kernel<E, DK, MODE>), dim3(pa.nprep + grid_p + ngate), dim3(64 * (4 + L::NP)),
                       lds, stream, (const E *)q, (const E *)k, (const E *)v, (const E *)g, (const E *)beta, S0,
                       (E *)o, S_T, snap.count > 0 || snap.packed ? snap.out : nullptr, snap.every_chunks,
                       snap.count, snap.packed ? 1 : 0, T, H, dv, nbh, nsl,
                       spin_limit < 0 ? kSpinLimit : spin_limit, fu.pub, og ? (const E *)og->gate : nullptr,
                       og ? og->w : nullptr, og ? og->eps : 0.f, grid_p, ngate, pa);
    return hipGetLastError();
}

// Workgroups of the plain prefill grid for these sizes.
int prefill_grid(int B, int H, int dv) { return ((B * H + kXCDs - 1) / kXCDs) * kXCDs * (dv / kVS); }

template <int MODE>
hipError_t launch_mode(const void *q, const void *k, const void *v, const void *g, const void *beta,
                       const float *S0, void *o, float *S_T, int B, int T, int H, int dk, int dv, bool fp32,
                       const Snapshots &snap, int spin_limit, const Fusion &fu, hipStream_t stream)
{
    if (fp32)
        return dk == 128 ? launch_ws<float, 128, MODE>(q, k, v, g, beta, S0, o, S_T, B, T, H, dv, snap, spin_limit,
                                                       fu, stream)
                         : launch_ws<float, 64, MODE>(q, k, v, g, beta, S0, o, S_T, B, T, H, dv, snap, spin_limit,
                                                      fu, stream);
    return dk == 128 ? launch_ws<__bf16, 128, MODE>(q, k, v, g, beta, S0, o, S_T, B, T, H, dv, snap, spin_limit,
                                                    fu, stream)
                     : launch_ws<__bf16, 64, MODE>(q, k, v, g, beta, S0, o, S_T, B, T, H, dv, snap, spin_limit,
                                                   fu, stream);
}

// T == 0: S_T = S0 (or 0).  One thread per state element.
__global__ void copy_state_kernel(const float *S0, float *S_T, long n)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        S_T[i] = S0 ? S0[i] : 0.f;
}

} // namespace

hipError_t launch_chunk16(const void *q, const void *k, const void *v, const void *g,
                          const void *beta, const float *S0, void *o, float *S_T, int B, int T,
                          int H, int dk, int dv, bool fp32, const Snapshots &snap, hipStream_t stream,
                          int spin_limit)
{
    return launch_mode<0>(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, fp32, snap, spin_limit, Fusion{}, stream);
}

hipError_t launch_chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *S0, void *o, float *S_T, int B, int T,
                            int H, int dk, int dv, bool fp32, const Snapshots &snap,
                            const FwdOptions &opt, hipStream_t stream)
{
    if ((long)B * H == 0)
        return hipSuccess;
    if (T == 0) {
        if (!S_T || S_T == S0)
            return hipSuccess;
        const long n = (long)B * H * dk * dv;
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           S0, S_T, n);
        return hipGetLastError();
    }
    return launch_chunk16(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, fp32, snap, stream, opt.spin_limit);
}

hipError_t launch_chunk_fwd_gated(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const float *S0, const OutputGate &og, void *y,
                                  float *S_T, int *pub, int B, int T, int H, int dk, int dv, bool fp32,
                                  const FwdOptions &opt, hipStream_t stream)
{
    if ((long)B * H == 0)
        return hipSuccess;
    const Snapshots none;
    if (T == 0)
        return launch_chunk_fwd(q, k, v, g, beta, S0, y, S_T, B, T, H, dk, dv, fp32, none, opt, stream);
    Fusion fu;
    fu.og = &og;
    fu.pub = pub;
    return launch_mode<1>(q, k, v, g, beta, S0, y, S_T, B, T, H, dk, dv, fp32, none, opt.spin_limit, fu, stream);
}

hipError_t launch_chunk_fwd_from_proj(const PrepInputs &pi, void *q, void *k, void *v, void *g, void *beta,
                                      const float *S0, void *o, float *S_T, int *done, int B, int T, int H,
                                      int dk, int dv, bool fp32, const FwdOptions &opt, hipStream_t stream)
{
    if ((long)B * H == 0)
        return hipSuccess;
    const Snapshots none;
    // fewer than kMinPrepCUs CUs left beside the prefill grid (or nothing to
    // prefill): the preprocessing pass, then the prefill -- the same arithmetic, so
    // the same bits.  The preprocessing streams its 2(3dk + dv) + 4 bytes per
    // token-head at about 20 GB/s per CU whether it runs alone or beside the
    // prefill, so it needs most of the chip to keep ahead: on B1 T65536 the fused
    // launch beats the two passes by 15 % with 128 CUs to spare (H64) and by 6 %
    // with 96 (H80), and takes 1.7 times as long with 64 (H96).
    if (T == 0 || prefill_grid(B, H, dv) > kCUs - kMinPrepCUs) {
        hipError_t e = launch_prefill_prep(pi.q_pre, pi.k_pre, pi.v_pre, pi.conv_w, pi.conv_init, pi.z, pi.A,
                                           pi.beta_logit, q, k, v, g, beta, pi.conv_final, B, T, H, dk, dv, fp32,
                                           stream);
        if (e != hipSuccess)
            return e;
        return launch_chunk_fwd(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, fp32, none, opt, stream);
    }
    Fusion fu;
    fu.prep = &pi;
    fu.done = done;
    return launch_mode<2>(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, fp32, none, opt.spin_limit, fu, stream);
}

} // namespace kda
