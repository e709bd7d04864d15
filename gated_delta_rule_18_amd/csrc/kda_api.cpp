// kda_api.cpp -- the C ABI declared in include/kda.h: argument validation,
// error mapping and dispatch to the HIP launchers.  No allocation and no host
// synchronisation; the only global state is the per-device address of the
// allocation-free backward's scratch array.
#include "kda.h"

#include <cstdint>

#include "kda_internal.h"

static_assert(kda::kNoallocScratchBytes == KDA_NOALLOC_SCRATCH_BYTES, "scratch size");

namespace {

// Largest batch or head count (each), and largest number of (sequence, head)
// pairs, of one prefill, preprocessing or backward call: grids and per-head
// byte strides stay inside 32-bit ranges.
constexpr int kMaxBH = 65535;
constexpr long long kMaxHeads = 1LL << 24;

bool aligned16(const void *p) { return (reinterpret_cast<std::uintptr_t>(p) & 15u) == 0; }
bool head_ok(int d) { return d == 64 || d == 128; }

bool overlap(const void *a, long long na, const void *b, long long nb)
{
    const char *x = reinterpret_cast<const char *>(a), *y = reinterpret_cast<const char *>(b);
    return a && b && x < y + nb && y < x + na;
}

// The checks every prefill entry shares (o: the output rows, o or y).
int check_fwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
              const float *S0, const void *o, const float *S_T, int B, int T, int H, int dk, int dv,
              int dtype)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return KDA_ERR_INVALID;
    if (dtype != KDA_BF16 && dtype != KDA_FP32)
        return KDA_ERR_INVALID;
    if (!head_ok(dk) || !head_ok(dv))
        return KDA_ERR_UNSUPPORTED;
    // index ranges of the kernel: 32-bit grids and per-head byte strides
    if (B > kMaxBH || H > kMaxBH || (long long)B * H > kMaxHeads)
        return KDA_ERR_INVALID;
    if ((long long)B * T * H * (dk > dv ? dk : dv) > (1LL << 40))
        return KDA_ERR_INVALID;
    const bool has_tokens = (long long)B * T * H > 0;
    if (has_tokens && (!q || !k || !v || !g || !beta || !o))
        return KDA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, g, o, S0, S_T};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return KDA_ERR_INVALID;
    // S_T may be S0 itself; a partial overlap would let one head's write race
    // with another head's read.
    const long long state_bytes = (long long)B * H * dk * dv * 4;
    if (S0 != S_T && overlap(S0, state_bytes, S_T, state_bytes))
        return KDA_ERR_INVALID;
    return KDA_OK;
}

int chunk_fwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
              const float *S0, void *o, float *S_T, int B, int T, int H, int dk, int dv, int dtype,
              int chunk, const kda::Snapshots &snap, const kda::FwdOptions &opt, void *stream)
{
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return KDA_ERR_INVALID;
    const int st = check_fwd(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, dtype);
    if (st != KDA_OK)
        return st;
    if (snap.out && !aligned16(snap.out))
        return KDA_ERR_INVALID;
    const long long state_bytes = (long long)B * H * dk * dv * 4;
    if (snap.count < 0)
        return KDA_ERR_INVALID;
    if (snap.count > 0) {
        if (!snap.out || snap.every_chunks <= 0 || (long long)snap.count * snap.every_chunks * chunk > T)
            return KDA_ERR_INVALID;
        const long long snap_bytes = state_bytes * snap.count;
        if (overlap(snap.out, snap_bytes, S0, state_bytes) || overlap(snap.out, snap_bytes, S_T, state_bytes))
            return KDA_ERR_INVALID;
    }
    // Every chunk size runs the 16-token kernel: the chunk size only changes how
    // the same map is blocked, and a 16-token chunk is already the 16-position
    // tile in which every decay factor stays bounded.  Snapshot spacing in its
    // chunks.
    kda::Snapshots ks = snap;
    ks.every_chunks = snap.every_chunks * (chunk / 16);
    hipError_t e = kda::launch_chunk_fwd(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv,
                                         dtype == KDA_FP32, ks, opt,
                                         reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int chunk_fwd_gated(const void *q, const void *k, const void *v, const void *g, const void *beta,
                    const float *S0, const void *gate, const float *norm_w, float eps, void *y, float *S_T,
                    void *workspace, size_t workspace_bytes, int B, int T, int H, int dk, int dv,
                    int dtype, const kda::FwdOptions &opt, void *stream)
{
    const int st = check_fwd(q, k, v, g, beta, S0, y, S_T, B, T, H, dk, dv, dtype);
    if (st != KDA_OK)
        return st;
    if (!(eps > 0.f) || !(eps < 1e30f))
        return KDA_ERR_INVALID;
    const long long rows = (long long)B * T * H;
    if (rows == 0)
        return kda::launch_chunk_fwd_gated(q, k, v, g, beta, S0, kda::OutputGate{}, y, S_T, nullptr, B, T, H,
                                           dk, dv, dtype == KDA_FP32, opt,
                                           reinterpret_cast<hipStream_t>(stream)) == hipSuccess
                   ? KDA_OK
                   : KDA_ERR_LAUNCH;
    const size_t need = kda_chunk_fwd_gated_workspace_size(B, H, dv);
    if (!gate || !aligned16(gate) || (norm_w && !aligned16(norm_w)) || !workspace || !aligned16(workspace) ||
        workspace_bytes < need)
        return KDA_ERR_INVALID;
    // y is written while the inputs are still being read: it may overlap none of
    // them, nor the workspace or the states
    const long long es = dtype == KDA_FP32 ? 4 : 2;
    const long long sb = (long long)B * H * dk * dv * 4;
    const void *in[] = {q, k, v, g, beta, gate, norm_w, S0, S_T};
    const long long in_n[] = {rows * dk * es, rows * dk * es, rows * dv * es, rows * dk * es, rows * es,
                              rows * dv * es, (long long)dv * 4, sb, sb};
    for (int j = 0; j < 9; ++j)
        if (overlap(y, rows * dv * es, in[j], in_n[j]) || overlap(workspace, (long long)need, in[j], in_n[j]))
            return KDA_ERR_INVALID;
    if (overlap(y, rows * dv * es, workspace, (long long)need))
        return KDA_ERR_INVALID;
    kda::OutputGate og;
    og.gate = gate;
    og.w = norm_w;
    og.eps = eps;
    hipError_t e = kda::launch_chunk_fwd_gated(q, k, v, g, beta, S0, og, y, S_T, static_cast<int *>(workspace), B,
                                               T, H, dk, dv, dtype == KDA_FP32, opt,
                                               reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int decode_step(const void *q_pre, const void *k_pre, const void *v_pre, const float *conv_w,
                void *conv_cache, int conv_pos, const void *g, const void *beta, float *S, void *o,
                int N, int H, int dk, int dv, int width, int dtype, const kda::OutputGate &og,
                void *stream)
{
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0 || conv_pos < 0)
        return KDA_ERR_INVALID;
    if (dtype != KDA_BF16 && dtype != KDA_FP32)
        return KDA_ERR_INVALID;
    if (width != 4)
        return KDA_ERR_INVALID;
    if (!head_ok(dk) || !head_ok(dv))
        return KDA_ERR_UNSUPPORTED;
    if ((long long)N * H == 0)
        return KDA_OK;
    if (!q_pre || !k_pre || !v_pre || !conv_w || !conv_cache || !g || !beta || !S || !o)
        return KDA_ERR_INVALID;
    const void *ptrs[] = {q_pre, k_pre, v_pre, conv_w, conv_cache, g, S, o};
    for (const void *p : ptrs)
        if (!aligned16(p))
            return KDA_ERR_INVALID;
    if ((long long)N * H > 0x7fffffffLL)
        return KDA_ERR_INVALID;
    hipError_t e = kda::launch_decode_step(q_pre, k_pre, v_pre, conv_w, conv_cache,
                                           conv_pos % (width - 1), g, beta, S, o, N, H, dk, dv,
                                           dtype == KDA_FP32, og, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int chunk_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
              const float *S0, const void *dO, const float *dS_T, float *dq, float *dk, float *dv,
              float *dg, float *dbeta, float *dS0, void *workspace, size_t workspace_bytes, int B,
              int T, int H, int dk_size, int dv_size, int dtype, void *stream, bool library_scratch,
              int xcd_flip = 0)
{
    if (B < 0 || T < 0 || H < 0 || dk_size <= 0 || dv_size <= 0)
        return KDA_ERR_INVALID;
    if (dtype != KDA_BF16 && dtype != KDA_FP32)
        return KDA_ERR_INVALID;
    if (!head_ok(dk_size) || !head_ok(dv_size))
        return KDA_ERR_UNSUPPORTED;
    if ((long long)B * T * H * (dk_size > dv_size ? dk_size : dv_size) > (1LL << 40) || B > kMaxBH ||
        H > kMaxBH || (long long)B * H > kMaxHeads)
        return KDA_ERR_INVALID;
    if ((long long)B * H == 0)
        return KDA_OK;
    const size_t need = kda_chunk_bwd_workspace_size(B, T, H, dk_size, dv_size);
    if (library_scratch) {
        if (need > kda::kNoallocScratchBytes)
            return KDA_ERR_TOO_LARGE;
    } else if (workspace_bytes < need || (need > 0 && !workspace) ||
               (reinterpret_cast<std::uintptr_t>(workspace) & 255u)) {
        return KDA_ERR_INVALID;
    }
    const bool has_tokens = T > 0;
    if (has_tokens && (!q || !k || !v || !g || !beta || !dO || !dq || !dk || !dv || !dg || !dbeta))
        return KDA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, g, beta, S0, dO, dS_T, dq, dk, dv, dg, dbeta, dS0};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return KDA_ERR_INVALID;
    if (library_scratch) {
        // the library's per-device array in place of a caller's workspace; its
        // address belongs to the current device, so the stream must too
        int cur = 0, sdev = 0;
        if (hipGetDevice(&cur) != hipSuccess ||
            hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess || cur != sdev)
            return KDA_ERR_INVALID;
        float *scratch = nullptr;
        if (kda::noalloc_scratch(&scratch) != hipSuccess)
            return KDA_ERR_LAUNCH;
        workspace = scratch;
    }
    const long long es = dtype == KDA_FP32 ? 4 : 2;
    const long long rows = (long long)B * T * H;
    const long long sb = (long long)B * H * dk_size * dv_size * 4;
    const void *in[] = {q, k, v, g, beta, S0, dO, dS_T, workspace};
    const long long in_n[] = {rows * dk_size * es, rows * dk_size * es, rows * dv_size * es,
                              rows * dk_size * es, rows * es, sb, rows * dv_size * es, sb,
                              (long long)need};
    const void *out[] = {dq, dk, dv, dg, dbeta, dS0};
    const long long out_n[] = {rows * dk_size * 4, rows * dk_size * 4, rows * dv_size * 4,
                               rows * dk_size * 4, rows * 4, sb};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 9; ++j)
            if (overlap(out[i], out_n[i], in[j], in_n[j]))
                return KDA_ERR_INVALID;
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out_n[i], out[j], out_n[j]))
                return KDA_ERR_INVALID;
    }
    hipError_t e = kda::launch_chunk_bwd(q, k, v, g, beta, S0, dO, dS_T, dq, dk, dv, dg, dbeta, dS0,
                                         static_cast<float *>(workspace), B, T, H, dk_size, dv_size,
                                         dtype == KDA_FP32, xcd_flip, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

} // namespace

extern "C" {

int kda_version(void) { return KDA_VERSION; }

const char *kda_strerror(int status)
{
    switch (status) {
    case KDA_OK:
        return "success";
    case KDA_ERR_INVALID:
        return "invalid argument (null pointer, bad size, dtype, chunk, width or misaligned buffer)";
    case KDA_ERR_UNSUPPORTED:
        return "unsupported head size (dk and dv must be 64 or 128)";
    case KDA_ERR_LAUNCH:
        return "HIP kernel launch failed";
    case KDA_ERR_TOO_LARGE:
        return "sizes need more workspace than the library's scratch array holds "
               "(KDA_NOALLOC_SCRATCH_BYTES)";
    default:
        return "unknown kda status";
    }
}

int kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                  const float *S0, void *o, float *S_T, int B, int T, int H, int dk, int dv,
                  int dtype, int chunk, void *stream)
{
    return chunk_fwd(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, dtype, chunk, kda::Snapshots{},
                     kda::FwdOptions{}, stream);
}

int kda_chunk_fwd_snapshots(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *S0, void *o, float *S_T, float *snaps,
                            int snap_every, int n_snaps, int B, int T, int H, int dk, int dv,
                            int dtype, int chunk, void *stream)
{
    return kda_chunk_fwd_ex(q, k, v, g, beta, S0, o, S_T, snaps, snap_every, n_snaps, B, T, H, dk, dv,
                            dtype, chunk, nullptr, stream);
}

int kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const void *g, const void *beta,
                     const float *S0, void *o, float *S_T, float *snaps, int snap_every, int n_snaps,
                     int B, int T, int H, int dk, int dv, int dtype, int chunk,
                     const kda_fwd_options *opts, void *stream)
{
    if (n_snaps < 0 || (n_snaps > 0 && (snap_every <= 0 || chunk <= 0 || snap_every % chunk != 0)))
        return KDA_ERR_INVALID;
    kda::Snapshots snap;
    if (n_snaps > 0) {
        if (!snaps)
            return KDA_ERR_INVALID;
        snap.out = snaps;
        snap.every_chunks = snap_every / chunk;
        snap.count = n_snaps;
    }
    kda::FwdOptions opt;
    if (opts) {
        if (opts->spin_limit < -1)
            return KDA_ERR_INVALID;
        opt.spin_limit = opts->spin_limit;
    }
    return chunk_fwd(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, dtype, chunk, snap, opt, stream);
}

size_t kda_chunk_fwd_gated_workspace_size(int B, int H, int dv)
{
    if (B < 0 || H < 0 || !head_ok(dv))
        return 0;
    return (size_t)B * H * (dv / 64) * 4 * sizeof(int);
}

int kda_chunk_fwd_gated(const void *q, const void *k, const void *v, const void *g, const void *beta,
                        const float *S0, const void *gate, const float *norm_w, float eps, void *y,
                        float *S_T, void *workspace, size_t workspace_bytes, int B, int T, int H, int dk,
                        int dv, int dtype, const kda_fwd_options *opts, void *stream)
{
    kda::FwdOptions opt;
    if (opts) {
        if (opts->spin_limit < -1)
            return KDA_ERR_INVALID;
        opt.spin_limit = opts->spin_limit;
    }
    return chunk_fwd_gated(q, k, v, g, beta, S0, gate, norm_w, eps, y, S_T, workspace, workspace_bytes, B, T,
                           H, dk, dv, dtype, opt, stream);
}

int kda_decode_step(const void *q_pre, const void *k_pre, const void *v_pre, const float *conv_w,
                    void *conv_cache, int conv_pos, const void *g, const void *beta, float *S,
                    void *o, int N, int H, int dk, int dv, int width, int dtype, void *stream)
{
    return decode_step(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S, o, N, H, dk,
                       dv, width, dtype, kda::OutputGate{}, stream);
}

int kda_decode_step_gated(const void *q_pre, const void *k_pre, const void *v_pre,
                          const float *conv_w, void *conv_cache, int conv_pos, const void *g,
                          const void *beta, float *S, const void *gate, const float *norm_w,
                          float eps, void *y, int N, int H, int dk, int dv, int width, int dtype,
                          void *stream)
{
    if (!(eps > 0.f) || !(eps < 1e30f))
        return KDA_ERR_INVALID;
    if ((long long)N * H > 0 && (!gate || !aligned16(gate) || (norm_w && !aligned16(norm_w))))
        return KDA_ERR_INVALID;
    kda::OutputGate og;
    og.gate = gate;
    og.w = norm_w;
    og.eps = eps;
    return decode_step(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S, y, N, H, dk,
                       dv, width, dtype, og, stream);
}

int kda_output_gate(const void *o, const void *gate, const float *norm_w, void *y, int rows, int H,
                    int dv, float eps, int dtype, void *stream)
{
    if (rows < 0 || H < 0 || dv <= 0 || !(eps > 0.f) || !(eps < 1e30f))
        return KDA_ERR_INVALID;
    if (dtype != KDA_BF16 && dtype != KDA_FP32)
        return KDA_ERR_INVALID;
    if (!head_ok(dv))
        return KDA_ERR_UNSUPPORTED;
    const long long units = (long long)rows * H;
    if (units == 0)
        return KDA_OK;
    if (!o || !gate || !y)
        return KDA_ERR_INVALID;
    const void *ptrs[] = {o, gate, y, norm_w};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return KDA_ERR_INVALID;
    // y may be o or gate itself (each element is read before it is written, by
    // the same lane); any other overlap is invalid
    const long long bytes = units * dv * (dtype == KDA_FP32 ? 4 : 2);
    if ((y != o && overlap(y, bytes, o, bytes)) || (y != gate && overlap(y, bytes, gate, bytes)))
        return KDA_ERR_INVALID;
    if (norm_w && overlap(y, bytes, norm_w, (long long)dv * 4))
        return KDA_ERR_INVALID;
    hipError_t e = kda::launch_output_gate(o, gate, norm_w, y, (long)units, dv, eps, dtype == KDA_FP32,
                                           reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int kda_validate_inputs(const void *g, const void *beta, long long *report, int B, int T, int H, int dk,
                        int dtype, void *stream)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0)
        return KDA_ERR_INVALID;
    if (dtype != KDA_BF16 && dtype != KDA_FP32)
        return KDA_ERR_INVALID;
    if (!report || (reinterpret_cast<std::uintptr_t>(report) & 7u) != 0)
        return KDA_ERR_INVALID;
    const long long nb = (long long)B * T * H, ng = nb * dk;
    if (ng > (1LL << 40))
        return KDA_ERR_INVALID;
    if (ng > 0 && (!g || !beta))
        return KDA_ERR_INVALID;
    hipError_t e = kda::launch_validate(g, beta, report, (long)ng, (long)nb, dtype == KDA_FP32,
                                        reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int kda_workgroup_xcds(int *xcd, int n, int lds_bytes, void *stream)
{
    if (n < 0 || n > (1 << 20) || lds_bytes < 0 || lds_bytes > 160 * 1024)
        return KDA_ERR_INVALID;
    if (n == 0)
        return KDA_OK;
    if (!xcd || (reinterpret_cast<std::uintptr_t>(xcd) & 3u) != 0)
        return KDA_ERR_INVALID;
    hipError_t e = kda::launch_workgroup_xcds(xcd, n, lds_bytes, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv)
{
    if (B < 0 || T < 0 || H < 0 || !head_ok(dk) || !head_ok(dv))
        return 0;
    if ((long long)B * T * H * (dk > dv ? dk : dv) > (1LL << 40))
        return 0;
    return kda::chunk_bwd_workspace_floats(B, T, H, dk, dv) * sizeof(float);
}

int kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                  const float *S0, const void *dO, const float *dS_T, float *dq, float *dk,
                  float *dv, float *dg, float *dbeta, float *dS0, void *workspace,
                  size_t workspace_bytes, int B, int T, int H, int dk_size, int dv_size, int dtype,
                  void *stream)
{
    return chunk_bwd(q, k, v, g, beta, S0, dO, dS_T, dq, dk, dv, dg, dbeta, dS0, workspace,
                     workspace_bytes, B, T, H, dk_size, dv_size, dtype, stream, false);
}

int kda_chunk_bwd_ex(const void *q, const void *k, const void *v, const void *g, const void *beta,
                     const float *S0, const void *dO, const float *dS_T, float *dq, float *dk,
                     float *dv, float *dg, float *dbeta, float *dS0, void *workspace,
                     size_t workspace_bytes, int B, int T, int H, int dk_size, int dv_size, int dtype,
                     const kda_bwd_options *opts, void *stream)
{
    return chunk_bwd(q, k, v, g, beta, S0, dO, dS_T, dq, dk, dv, dg, dbeta, dS0, workspace,
                     workspace_bytes, B, T, H, dk_size, dv_size, dtype, stream, false,
                     opts && opts->fail_xcd_check ? 1 : 0);
}

int kda_chunk_bwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                          const void *beta, const float *S0, const void *dO, const float *dS_T,
                          float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0, int B,
                          int T, int H, int dk_size, int dv_size, int dtype, void *stream)
{
    return chunk_bwd(q, k, v, g, beta, S0, dO, dS_T, dq, dk, dv, dg, dbeta, dS0, nullptr, 0, B, T,
                     H, dk_size, dv_size, dtype, stream, true);
}

} // extern "C"

namespace {

// The checks of the preprocessing's arguments (shared by kda_prefill_prep and
// kda_chunk_fwd_from_proj).  KDA_OK with B*H == 0 means there is nothing to do.
int check_prep(const void *q_pre, const void *k_pre, const void *v_pre, const float *conv_w,
               const void *conv_init, const void *z, const float *A, const void *beta_logit, void *q, void *k,
               void *v, void *g, void *beta, void *conv_final, int B, int T, int H, int dk, int dv, int width,
               int dtype)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return KDA_ERR_INVALID;
    if (dtype != KDA_BF16 && dtype != KDA_FP32)
        return KDA_ERR_INVALID;
    if (width != 4)
        return KDA_ERR_INVALID;
    if (!head_ok(dk) || !head_ok(dv))
        return KDA_ERR_UNSUPPORTED;
    if ((long long)B * T * H * (dk > dv ? dk : dv) > (1LL << 40) || B > kMaxBH || H > kMaxBH ||
        (long long)B * H > kMaxHeads)
        return KDA_ERR_INVALID;
    if ((long long)B * H == 0)
        return KDA_OK;
    if (!conv_w || !A)
        return KDA_ERR_INVALID;
    const bool has_tokens = T > 0;
    if (has_tokens && (!q_pre || !k_pre || !v_pre || !z || !beta_logit || !q || !k || !v || !g || !beta))
        return KDA_ERR_INVALID;
    const void *ptrs[] = {q_pre, k_pre, v_pre, conv_w, conv_init, z, q, k, v, g, conv_final};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return KDA_ERR_INVALID;
    const long long es = dtype == KDA_FP32 ? 4 : 2;
    const long long nk = (long long)B * T * H * dk * es, nv = (long long)B * T * H * dv * es;
    const long long nb = (long long)B * T * H * es, nc = (long long)B * H * (width - 1) * (2 * dk + dv) * es;
    const void *in[] = {q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit};
    const long long in_n[] = {nk, nk, nv, (long long)H * (2 * dk + dv) * width * 4, nc, nk, (long long)H * 4, nb};
    const void *out[] = {q, k, v, g, beta, conv_final};
    const long long out_n[] = {nk, nk, nv, nk, nb, nc};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 8; ++j)
            if (!(i == 5 && j == 4 && out[i] == in[j]) && overlap(out[i], out_n[i], in[j], in_n[j]))
                return KDA_ERR_INVALID;
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out_n[i], out[j], out_n[j]))
                return KDA_ERR_INVALID;
    }
    return KDA_OK;
}

} // namespace

extern "C" {

int kda_prefill_prep(const void *q_pre, const void *k_pre, const void *v_pre, const float *conv_w,
                     const void *conv_init, const void *z, const float *A, const void *beta_logit,
                     void *q, void *k, void *v, void *g, void *beta, void *conv_final, int B, int T,
                     int H, int dk, int dv, int width, int dtype, void *stream)
{
    const int st = check_prep(q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit, q, k, v, g, beta,
                              conv_final, B, T, H, dk, dv, width, dtype);
    if (st != KDA_OK || (long long)B * H == 0)
        return st;
    hipError_t e = kda::launch_prefill_prep(q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit,
                                            q, k, v, g, beta, conv_final, B, T, H, dk, dv,
                                            dtype == KDA_FP32, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

size_t kda_chunk_fwd_from_proj_workspace_size(int B, int T, int H)
{
    if (B < 0 || T < 0 || H < 0)
        return 0;
    return (size_t)B * H * (((size_t)T + 127) / 128) * sizeof(int);
}

int kda_chunk_fwd_from_proj(const void *q_pre, const void *k_pre, const void *v_pre, const float *conv_w,
                            const void *conv_init, const void *z, const float *A, const void *beta_logit,
                            void *q, void *k, void *v, void *g, void *beta, void *conv_final, const float *S0,
                            void *o, float *S_T, void *workspace, size_t workspace_bytes, int B, int T, int H,
                            int dk, int dv, int width, int dtype, const kda_fwd_options *opts, void *stream)
{
    int st = check_prep(q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit, q, k, v, g, beta, conv_final,
                        B, T, H, dk, dv, width, dtype);
    if (st != KDA_OK)
        return st;
    st = check_fwd(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, dtype);
    if (st != KDA_OK)
        return st;
    kda::FwdOptions opt;
    if (opts) {
        if (opts->spin_limit < -1)
            return KDA_ERR_INVALID;
        opt.spin_limit = opts->spin_limit;
    }
    if ((long long)B * H == 0)
        return KDA_OK;
    const size_t need = kda_chunk_fwd_from_proj_workspace_size(B, T, H);
    if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
        return KDA_ERR_INVALID;
    // o, S_T and the workspace are written while everything else is read or written
    const long long es = dtype == KDA_FP32 ? 4 : 2;
    const long long rows = (long long)B * T * H;
    const long long nk = rows * dk * es, nv = rows * dv * es, sb = (long long)B * H * dk * dv * 4;
    const long long nc = (long long)B * H * (width - 1) * (2 * dk + dv) * es;
    const void *all[] = {q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit, q, k, v, g, beta, conv_final, S0};
    const long long all_n[] = {nk, nk, nv, (long long)H * (2 * dk + dv) * width * 4, nc, nk, (long long)H * 4,
                               rows * es, nk, nk, nv, nk, rows * es, nc, sb};
    // the preprocessing's outputs (checked against its inputs above) against S0
    for (int j = 8; j < 14; ++j)
        if (overlap(all[j], all_n[j], S0, sb))
            return KDA_ERR_INVALID;
    const void *out[] = {o, S_T, workspace};
    const long long out_n[] = {nv, sb, (long long)need};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 15; ++j)
            if (!(i == 1 && j == 14 && out[i] == all[j]) && overlap(out[i], out_n[i], all[j], all_n[j]))
                return KDA_ERR_INVALID;
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out_n[i], out[j], out_n[j]))
                return KDA_ERR_INVALID;
    }
    kda::PrepInputs pi;
    pi.q_pre = q_pre;
    pi.k_pre = k_pre;
    pi.v_pre = v_pre;
    pi.z = z;
    pi.beta_logit = beta_logit;
    pi.conv_init = conv_init;
    pi.conv_w = conv_w;
    pi.A = A;
    pi.conv_final = conv_final;
    hipError_t e = kda::launch_chunk_fwd_from_proj(pi, q, k, v, g, beta, S0, o, S_T, static_cast<int *>(workspace),
                                                   B, T, H, dk, dv, dtype == KDA_FP32, opt,
                                                   reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

} // extern "C"
