// kda_internal.h -- host-side launch entry points of the KDA kernels.  Only the
// C-ABI layer (kda_api.cpp) calls these; arguments are validated there.
#pragma once
#include <hip/hip_runtime.h>

namespace kda {

// Intermediate states a prefill writes: snapshot s (s < count) is the state
// after the first (s + 1) * every_chunks chunks, at out + s * B*H*dk*dv.
// packed (chunk-16 kernel only; the backward's private workspace): the initial
// state comes first (snapshot s then sits at out + (s + 1) * B*H*dk*dv), the
// states are stored in the element type instead of fp32, and each head's state
// in 4-row groups, element (r, c) at ((r / 4) * dv + c) * 4 + r % 4 -- one
// contiguous 4-element piece per accumulator lane of the writer.
struct Snapshots {
    float *out = nullptr;
    int every_chunks = 0;
    int count = 0;
    bool packed = false;
};

// Knobs of a prefill launch that callers other than tests leave at their
// defaults.  spin_limit: polls before an internal hand-off wait gives up and the
// workgroup marks its results NaN (< 0 = the built-in limit).
struct FwdOptions {
    int spin_limit = -1;
};

// Every chunk size the C ABI accepts runs the 16-token kernel
// (kda_prefill_ws.hip); snap.every_chunks counts 16-token chunks.
hipError_t launch_chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *S0, void *o, float *S_T,
                            int B, int T, int H, int dk, int dv, bool fp32,
                            const Snapshots &snap, const FwdOptions &opt, hipStream_t stream);

// The 16-token kernel itself (T > 0, B*H > 0).
hipError_t launch_chunk16(const void *q, const void *k, const void *v, const void *g,
                          const void *beta, const float *S0, void *o, float *S_T,
                          int B, int T, int H, int dk, int dv, bool fp32, const Snapshots &snap,
                          hipStream_t stream, int spin_limit = -1);

// Debug check of the value domains: report (device int64[4]) receives the number
// of g outside [-5, 0] (or NaN), the first such flat index (-1 if none), and the
// same two for beta outside [0, 1]; ng, nb are the element counts.
hipError_t launch_validate(const void *g, const void *beta, long long *report, long ng, long nb, bool fp32,
                           hipStream_t stream);

// Output exposure gate fused into the decode step: when gate is not null the
// step writes y = Sigmoid(gate) * o / sqrt(mean o^2 + eps) * w in place of o
// (w null = ones).
struct OutputGate {
    const void *gate = nullptr;
    const float *w = nullptr;
    float eps = 0.f;
};

hipError_t launch_decode_step(const void *q_pre, const void *k_pre, const void *v_pre,
                              const float *conv_w, void *conv_cache, int oldest_slot,
                              const void *g, const void *beta, float *S, void *o,
                              int N, int H, int dk, int dv, bool fp32, const OutputGate &og,
                              hipStream_t stream);

// The prefill with the output exposure gate fused (kda_chunk_fwd_gated): y
// receives Sigmoid(gate) * o / sqrt(mean o^2 + eps) * w per (token, head) in
// place of o; pub holds B * H * (dv / 64) * 4 ints of scratch (the consumers'
// progress words, cleared by the launch).
hipError_t launch_chunk_fwd_gated(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const float *S0, const OutputGate &og, void *y,
                                  float *S_T, int *pub, int B, int T, int H, int dk, int dv, bool fp32,
                                  const FwdOptions &opt, hipStream_t stream);

// The prefill with the preprocessing fused (kda_chunk_fwd_from_proj): the
// pre-activations of kda_prefill_prep in, its outputs q, k, v, g, beta (written,
// then read by the prefill in the same launch), o and S_T out.  done holds
// B * H * ceil(T / 128) ints of scratch (tile flags, cleared by the launch).
struct PrepInputs {
    const void *q_pre = nullptr, *k_pre = nullptr, *v_pre = nullptr, *z = nullptr, *beta_logit = nullptr,
               *conv_init = nullptr;
    const float *conv_w = nullptr, *A = nullptr;
    void *conv_final = nullptr;
};
hipError_t launch_chunk_fwd_from_proj(const PrepInputs &pi, void *q, void *k, void *v, void *g, void *beta,
                                      const float *S0, void *o, float *S_T, int *done, int B, int T, int H,
                                      int dk, int dv, bool fp32, const FwdOptions &opt, hipStream_t stream);

// Backward pass: gradients (fp32) of <dO, o> + <dS_T, S_T> through kda_chunk_fwd.
// workspace holds chunk_bwd_workspace_floats(...) floats.
size_t chunk_bwd_workspace_floats(int B, int T, int H, int dk, int dv);
hipError_t launch_chunk_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                            const float *S0, const void *dO, const float *dST, float *dq, float *dk,
                            float *dv, float *dg, float *dbeta, float *dS0, float *workspace, int B, int T,
                            int H, int DK, int DV, bool fp32, int xcd_flip, hipStream_t stream);

// The library's own backward workspace, for callers that cannot allocate: a
// device array of kNoallocScratchBytes in every GPU's memory (one copy per
// device, held until the process ends).  noalloc_scratch returns the current
// device's copy, looked up once per device.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(float **ptr);

// Debug: workgroup i of an n-workgroup launch, each requesting lds_bytes of
// dynamic LDS, writes the XCD it ran on to xcd[i].
hipError_t launch_workgroup_xcds(int *xcd, int n, int lds_bytes, hipStream_t stream);

// The output exposure gate alone over `units` (row, head) rows of dv elements.
hipError_t launch_output_gate(const void *o, const void *gate, const float *w, void *y, long units,
                              int dv, float eps, bool fp32, hipStream_t stream);

hipError_t launch_prefill_prep(const void *q_pre, const void *k_pre, const void *v_pre,
                               const float *conv_w, const void *conv_init, const void *z,
                               const float *A, const void *beta_logit, void *q, void *k, void *v,
                               void *g, void *beta, void *conv_final, int B, int T, int H, int dk,
                               int dv, bool fp32, hipStream_t stream);

} // namespace kda
