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
// once.  A workgroup of four wavefronts owns two heads (h0, h0 + 1) of one
// sequence over a kTT-token tile (the unit of kda_prep_unit.h, which holds the
// arithmetic).  Workgroups are numbered head pair first, so the workgroups in
// flight at any time cover whole token rows of every tensor (all heads of the
// same tokens) and the device reads and writes long contiguous runs instead of
// 512-byte pieces scattered over the sequence.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_prep_unit.h"

namespace kda {
namespace {

constexpr int kU = 8;                    // tokens loaded ahead

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void prep_kernel(
    const E *__restrict__ q_pre, const E *__restrict__ k_pre, const E *__restrict__ v_pre,
    const float *__restrict__ conv_w, const E *conv_init, const E *__restrict__ z,
    const float *__restrict__ A, const E *__restrict__ beta_logit, E *__restrict__ q,
    E *__restrict__ k, E *__restrict__ v, E *__restrict__ g, E *__restrict__ beta, E *conv_final,
    int T, int H)
{
    // head pair fastest (one-dimensional numbering: no 65535 limit on tiles)
    const int npairs = (H + 1) / 2;
    const int hp = (int)(blockIdx.x % npairs), tile = (int)(blockIdx.x / npairs), b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int bhA = b * H + 2 * hp, bhB = 2 * hp + 1 < H ? bhA + 1 : -1;
    prep_unit<E, DK, DV, kU>(q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit, q, k, v, g, beta,
                             conv_final, T, H, bhA, bhB, tile, wave, lane);
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
    hipLaunchKernelGGL((prep_kernel<E, DK, DV>), dim3((unsigned)(((H + 1) / 2) * (long)tiles), 1, B), dim3(256), 0, stream,
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
