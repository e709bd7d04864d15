/*
 * kda.h -- C ABI of libkda.so: the Kimi Delta Attention (KDA) layer recurrence
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读",
 * section 3.1, KDA recurrence equation; restated on page "Kimi K3 架构篇：一文详解
 * 2.8 万亿参数的巨型怪兽", section "KDA 到底在算什么"): per head, with state
 * S_t in R^{dk x dv} (row = key channel, column = value channel),
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 *
 * where alpha_t = exp(g_t) per key channel and g_t lies in [g_min, 0] with
 * g_min = -5 (same page, section 3.3, lower-bounded decay equation).  The
 * query is not scaled.
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers, row-major and contiguous, with
 *     16-byte aligned base addresses.  The caller allocates and frees them; the
 *     library allocates nothing and keeps no global state, so concurrent calls
 *     on different buffers are safe -- except kda_chunk_bwd_noalloc, which
 *     works in a device array the library holds (one per GPU).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it; the call returns without synchronising.  Kernel
 *     faults surface on the stream, not in the return code; a prefill whose
 *     internal hand-off gives up marks its outputs NaN (kda_chunk_fwd_ex).
 *   - dtype KDA_BF16: q, k, v, g, beta, o (and the decode conv cache) are
 *     bfloat16; the state is fp32.  dtype KDA_FP32 (test mode): every tensor is
 *     fp32.
 *   - Return 0 on success or a negative KDA_ERR_* code; nothing is enqueued
 *     when a code other than KDA_ERR_LAUNCH is returned.
 *   - Values outside the stated domains (g outside [-5, 0], beta outside
 *     [0, 1], non-finite inputs) are not diagnosed by the compute entry points
 *     and give unspecified output; kda_validate_inputs reports them.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 150 /* 1.5.0 */

enum kda_dtype {
    KDA_BF16 = 0, /* bf16 activations, fp32 state */
    KDA_FP32 = 1  /* everything fp32 (test mode) */
};

enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID = -1,     /* null required pointer, bad size, bad dtype/chunk/width/misalignment */
    KDA_ERR_UNSUPPORTED = -2, /* a head size the library has no kernel for (dk, dv not in {64, 128}) */
    KDA_ERR_LAUNCH = -3,      /* the HIP runtime rejected the launch */
    KDA_ERR_TOO_LARGE = -4    /* kda_chunk_bwd_noalloc: the sizes need more than its scratch array */
};

/*
 * kda_chunk_fwd -- chunkwise-parallel prefill of one KDA layer.
 *
 * Defines (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读",
 * section 3.3, chunk-interface equation): the sequence is cut into chunks of
 * `chunk` tokens processed in parallel inside a chunk, and the state leaving
 * chunk c is the state entering chunk c+1.  The result equals the token-serial
 * recurrence above up to floating-point association order.
 *
 *   q, k, g : [B, T, H, dk]   (dtype)    queries, keys (normally unit length), log-decay g
 *   v       : [B, T, H, dv]   (dtype)    values
 *   beta    : [B, T, H]       (dtype)    write strength
 *   S0      : [B, H, dk, dv]  fp32       initial state; NULL means zero
 *   o       : [B, T, H, dv]   (dtype)    output, o_t = S_t^T q_t (written)
 *   S_T     : [B, H, dk, dv]  fp32       final state (written); NULL = not returned.
 *                                        S_T may equal S0 (in-place streaming over
 *                                        segments); any other overlap is invalid.
 *   dk, dv  : 64 or 128
 *   B, H    : each at most 65535, and B*H at most 2^24
 *   chunk   : 16, 32 or 64 tokens per chunk.  Every size runs the same kernel,
 *             which works on 16-token chunks -- the 16-position tile of section
 *             3.3 inside which every decay factor stays bounded -- so the
 *             results are identical bit for bit; `chunk` only sets the unit of
 *             snapshot spacing (kda_chunk_fwd_snapshots).
 * T may be any value >= 0 (a ragged last chunk is handled); T == 0 copies S0
 * to S_T (or zeroes S_T when S0 is NULL).
 * The kernel's parts hand work to each other through bounded waits; should
 * one ever give up, the affected outputs are NaN (see kda_chunk_fwd_ex).
 */
int kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                  const void *beta, const float *S0, void *o, float *S_T,
                  int B, int T, int H, int dk, int dv, int dtype, int chunk,
                  void *stream);

/*
 * kda_chunk_fwd_snapshots -- kda_chunk_fwd that also writes intermediate states.
 *
 * Defines (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读",
 * section 9, the figure on the KDA-checkpoint / MLA-hash-block prefix cache):
 * a KDA layer keeps one recurrent state per sequence, so a cached prefix can
 * only be resumed at token counts where that state was saved; the pages save
 * it every 512 tokens.  Snapshot s is the state after the first
 * (s + 1) * snap_every tokens -- exactly the S_T a kda_chunk_fwd over that
 * prefix returns, and a valid S0 to continue from there.
 *
 * Arguments as kda_chunk_fwd, plus
 *   snaps      : [n_snaps, B, H, dk, dv] fp32 (written); snaps + s*B*H*dk*dv is
 *                snapshot s.  May be NULL when n_snaps == 0.  Must not overlap
 *                S0 or S_T.
 *   snap_every : tokens between snapshots, a positive multiple of `chunk`
 *   n_snaps    : >= 0 with n_snaps * snap_every <= T
 * Errors: KDA_ERR_INVALID for a violated condition above, else as kda_chunk_fwd.
 * Cost: 4*dk*dv bytes written per head per snapshot on top of kda_chunk_fwd.
 */
int kda_chunk_fwd_snapshots(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *S0, void *o, float *S_T,
                            float *snaps, int snap_every, int n_snaps,
                            int B, int T, int H, int dk, int dv, int dtype, int chunk,
                            void *stream);

/*
 * kda_chunk_fwd_ex -- kda_chunk_fwd_snapshots with the library's internal
 * limits exposed; for tests and debugging.  (Same page, section 3.3, chunk
 * interface; the options change no result, only how failures of the kernel's
 * internal hand-offs are handled.)
 *
 * Arguments as kda_chunk_fwd_snapshots, plus
 *   opts : NULL = defaults (what kda_chunk_fwd uses), else
 *     spin_limit : number of polls after which a wait of one part of a
 *                  workgroup for another gives up; -1 = the built-in limit
 *                  (about 0.1 s of waiting, which normal operation never
 *                  comes near), 0 = give up at the first unsatisfied poll.
 * When a wait gives up the kernel does not hang: it finishes, and it writes NaN
 * in place of the o rows of every chunk from the one at which the workgroup
 * noticed on, of the (head, value slice)'s part of S_T, and of any snapshot
 * taken after that point.  Values written before are exact results.
 * Errors: as kda_chunk_fwd_snapshots; KDA_ERR_INVALID for spin_limit < -1.
 */
typedef struct kda_fwd_options {
    int spin_limit;
} kda_fwd_options;

int kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, const float *S0, void *o, float *S_T,
                     float *snaps, int snap_every, int n_snaps,
                     int B, int T, int H, int dk, int dv, int dtype, int chunk,
                     const kda_fwd_options *opts, void *stream);

/*
 * kda_decode_step -- one generated token of one KDA layer for N sequences.
 *
 * Defines (same page, section 3.2): the decode interface
 * (x_t, S_{t-1}, C^conv_{t-1}) -> (y_t, S_t, C^conv_t), the input branches
 * q, k = L2Norm(Swish(ShortConv(W x))), v = Swish(ShortConv(W_v x)), and the
 * step order Sbar = Diag(alpha) S, vhat = Sbar^T k, S = Sbar + beta k (v - vhat)^T,
 * o = S^T q (read after the write).  The projections W x are done by the
 * caller; this call starts from their outputs.  Readings where the pages are
 * silent: ShortConv is depthwise and causal with no bias, tap 0 multiplies
 * the oldest token; Swish(u) = u * sigmoid(u); L2Norm(x) = x / sqrt(sum x^2 + 1e-6).
 *
 *   q_pre, k_pre : [N, H, dk]  (dtype)   projected pre-activations of x_t
 *   v_pre        : [N, H, dv]  (dtype)
 *   conv_w       : [H, 2dk+dv, width] fp32   taps, channel order q | k | v
 *   conv_cache   : [N, H, width-1, 2dk+dv] (dtype), a ring of the previous
 *                  width-1 pre-activations; slot (conv_pos mod (width-1)) holds
 *                  the oldest and is overwritten with x_t (read and written)
 *   conv_pos     : >= 0; the caller advances it by one per step
 *   g            : [N, H, dk] (dtype)     log-decay of this step
 *   beta         : [N, H]     (dtype)
 *   S            : [N, H, dk, dv] fp32    state, updated in place
 *   o            : [N, H, dv] (dtype)     output o_t = S_t^T q_t (written)
 *   width        : 4
 *   dk, dv       : 64 or 128
 */
int kda_decode_step(const void *q_pre, const void *k_pre, const void *v_pre,
                    const float *conv_w, void *conv_cache, int conv_pos,
                    const void *g, const void *beta, float *S, void *o,
                    int N, int H, int dk, int dv, int width, int dtype,
                    void *stream);

/*
 * kda_prefill_prep -- prefill preprocessing: projected pre-activations to the
 * q, k, v, g, beta that kda_chunk_fwd consumes.
 *
 * Defines (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读",
 * section 3.2, input-branch equations, applied to every token of a sequence;
 * section 3.3, lower-bounded decay equation):
 *   q_t = L2Norm(Swish(ShortConv(q_pre)_t)),  k_t likewise,
 *   v_t = Swish(ShortConv(v_pre)_t),
 *   beta_t = Sigmoid(beta_logit_t),
 *   g_t = -5 * Sigmoid(e^{A[h]} * z_t)       (so g lies in (-5, 0) by construction)
 * with the ShortConv, Swish and L2Norm readings of kda_decode_step.  The conv
 * window of the first tokens reaches into `conv_init`, the 3 pre-activations
 * before token 0; the call returns in `conv_final` the last 3, so a following
 * prefill segment (conv_init = conv_final) or a decode loop (conv_cache =
 * conv_final with conv_pos = 0) continues the sequence.
 *
 *   q_pre, k_pre, z : [B, T, H, dk]  (dtype)   projections; z feeds the gate
 *   v_pre           : [B, T, H, dv]  (dtype)
 *   conv_w          : [H, 2dk+dv, width] fp32  taps, channel order q | k | v, tap 0 = oldest
 *   conv_init       : [B, H, width-1, 2dk+dv] (dtype), oldest first; NULL = zero history
 *   A               : [H] fp32                 per-head gate scale exponent A^h
 *   beta_logit      : [B, T, H]      (dtype)
 *   q, k, g         : [B, T, H, dk]  (dtype)   written
 *   v               : [B, T, H, dv]  (dtype)   written
 *   beta            : [B, T, H]      (dtype)   written
 *   conv_final      : [B, H, width-1, 2dk+dv] (dtype), written, oldest first; NULL = not
 *                     returned.  May equal conv_init (in-place streaming); no other
 *                     output may overlap an input.
 *   width           : 4;  dk, dv : 64 or 128
 * Errors: KDA_ERR_INVALID (null required pointer, bad size/width/dtype,
 * misaligned buffer, overlapping buffers), KDA_ERR_UNSUPPORTED, KDA_ERR_LAUNCH.
 * conv_w and A are required whenever B*H > 0; the sequence tensors when B*T*H > 0.
 */
int kda_prefill_prep(const void *q_pre, const void *k_pre, const void *v_pre,
                     const float *conv_w, const void *conv_init, const void *z,
                     const float *A, const void *beta_logit,
                     void *q, void *k, void *v, void *g, void *beta, void *conv_final,
                     int B, int T, int H, int dk, int dv, int width, int dtype,
                     void *stream);

/*
 * kda_chunk_fwd_from_proj -- kda_prefill_prep and kda_chunk_fwd in one launch:
 * from the projected pre-activations to o and S_T.
 *
 * Defines (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section
 * 3.2, input-branch equations, and section 3.3, lower-bounded decay equation,
 * as kda_prefill_prep; then section 3.3, chunk interface, as kda_chunk_fwd):
 * every output is bit for bit what kda_prefill_prep followed by kda_chunk_fwd
 * writes.  Workgroups of the launch on the CUs the prefill leaves idle run the
 * preprocessing tile by tile (128 tokens), ahead of the prefill workgroups,
 * which read each tile once its flag is set.  When the prefill leaves fewer
 * than 96 of the 256 CUs idle (B*H*(dv/64), rounded up to a multiple of 8, above
 * 160 workgroups) the preprocessing would fall behind, and the call runs the
 * two passes one after the other instead.
 *
 * Arguments: those of kda_prefill_prep (q, k, v, g, beta and conv_final are
 * written, and q, k, v, g, beta are then the prefill's inputs), then
 *   S0, o, S_T : as kda_chunk_fwd (S_T may equal S0)
 *   workspace  : device memory of at least
 *                kda_chunk_fwd_from_proj_workspace_size(B, T, H) bytes (one flag
 *                per (sequence, head, 128-token tile)), 16-byte aligned, owned by
 *                the caller; contents before and after the call do not matter.
 *                Calls that may run at the same time need separate workspaces.
 *   opts       : NULL = defaults, else as kda_chunk_fwd_ex (spin_limit also bounds
 *                the prefill's waits for the preprocessing; a prefill workgroup
 *                whose tile flag shows a preprocessing workgroup on another XCD --
 *                the launch assumes workgroups i and i + 8 share an XCD -- marks
 *                its outputs NaN like a wait that gave up)
 * Errors: as kda_prefill_prep and kda_chunk_fwd; KDA_ERR_INVALID also for a null,
 * misaligned or short workspace, spin_limit < -1, or o, S_T or the workspace
 * overlapping any other buffer (S_T = S0 allowed).
 */
int kda_chunk_fwd_from_proj(const void *q_pre, const void *k_pre, const void *v_pre,
                            const float *conv_w, const void *conv_init, const void *z,
                            const float *A, const void *beta_logit,
                            void *q, void *k, void *v, void *g, void *beta, void *conv_final,
                            const float *S0, void *o, float *S_T,
                            void *workspace, size_t workspace_bytes,
                            int B, int T, int H, int dk, int dv, int width, int dtype,
                            const kda_fwd_options *opts, void *stream);

/* Bytes of workspace kda_chunk_fwd_from_proj needs (0 for invalid sizes). */
size_t kda_chunk_fwd_from_proj_workspace_size(int B, int T, int H);

/*
 * kda_output_gate -- the output exposure gate of a KDA layer, before W_o.
 *
 * Defines (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读",
 * section 3.2, output equation y_t = W_o[Sigmoid(W_g x_t) (.) RMSNorm(o~_t)]):
 * the bracket, with RMSNorm over the dv channels of each (row, head) -- the
 * section says it steadies each head's readout -- and a per-channel weight
 * shared by the heads:
 *     y[r,h,c] = Sigmoid(gate[r,h,c]) * o[r,h,c] / sqrt(mean_c' o[r,h,c']^2 + eps) * w[c]
 * W_g x_t (`gate`) and W_o are the caller's GEMMs.  This is the epilogue for
 * kda_chunk_fwd's output; kda_decode_step_gated fuses it into decode.
 *
 *   o      : [rows, H, dv] (dtype)   readout o~ (e.g. kda_chunk_fwd's o, rows = B*T)
 *   gate   : [rows, H, dv] (dtype)   gate pre-activation W_g x_t
 *   norm_w : [dv] fp32               RMSNorm weight; NULL = all ones
 *   y      : [rows, H, dv] (dtype)   written; may be o itself or gate itself
 *                                    (in place), any other overlap is invalid
 *   eps    : > 0 (1e-6 is the reading used by the tests)
 *   dv     : 64 or 128
 * Errors: KDA_ERR_INVALID (null/misaligned pointer, bad size or eps, overlap),
 * KDA_ERR_UNSUPPORTED (dv), KDA_ERR_LAUNCH.
 */
int kda_output_gate(const void *o, const void *gate, const float *norm_w, void *y,
                    int rows, int H, int dv, float eps, int dtype, void *stream);

/*
 * kda_decode_step_gated -- kda_decode_step with the output exposure gate fused:
 * the step writes y = Sigmoid(gate) * RMSNorm(o~) * w (as kda_output_gate
 * defines it, same page, section 3.2, output equation) in place of o~, so the
 * readout never goes through HBM.  The state and the conv cache are updated
 * exactly as kda_decode_step updates them.
 *
 * Arguments as kda_decode_step, with o replaced by
 *   gate   : [N, H, dv] (dtype)   gate pre-activation W_g x_t of this step
 *   norm_w : [dv] fp32            RMSNorm weight; NULL = all ones
 *   eps    : > 0
 *   y      : [N, H, dv] (dtype)   written
 * Errors: as kda_decode_step; KDA_ERR_INVALID also for a null or misaligned
 * gate, a misaligned norm_w or a bad eps.
 */
int kda_decode_step_gated(const void *q_pre, const void *k_pre, const void *v_pre,
                          const float *conv_w, void *conv_cache, int conv_pos,
                          const void *g, const void *beta, float *S,
                          const void *gate, const float *norm_w, float eps, void *y,
                          int N, int H, int dk, int dv, int width, int dtype,
                          void *stream);

/*
 * kda_chunk_fwd_gated -- kda_chunk_fwd with the output exposure gate fused: the
 * call writes y = Sigmoid(gate) * RMSNorm(o~) * w (as kda_output_gate defines
 * it, page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section 3.2,
 * output equation) for every (token, head), bit for bit what kda_chunk_fwd
 * followed by kda_output_gate writes.  The prefill writes each 16-token block
 * of o~ into y, and workgroups of the same launch, on CUs the prefill leaves
 * idle, gate the block in place once both value halves of its head are there,
 * reading it back from the L2 rather than from HBM.
 *
 * Arguments as kda_chunk_fwd (the 16-token kernel; there is no chunk argument),
 * with o replaced by
 *   gate      : [B, T, H, dv] (dtype)   gate pre-activation W_g x_t
 *   norm_w    : [dv] fp32               RMSNorm weight; NULL = all ones
 *   eps       : > 0
 *   y         : [B, T, H, dv] (dtype)   written; must not overlap any other buffer
 *   workspace : device memory of at least kda_chunk_fwd_gated_workspace_size(B, H, dv)
 *               bytes (the prefill's progress counters), 16-byte aligned, owned by
 *               the caller; its contents before the call do not matter and after it
 *               are unspecified.  Calls that may run at the same time need separate
 *               workspaces.
 *   opts      : NULL = defaults, else as kda_chunk_fwd_ex; spin_limit bounds the
 *               gate's waits for the prefill too, and a block whose wait gave up
 *               is written as NaN.  The hand-off assumes workgroups i and i + 8
 *               share an XCD (so that its L2 holds what it reads); a block whose
 *               progress words show another XCD is written as NaN too.
 * Errors: as kda_chunk_fwd; KDA_ERR_INVALID also for a null or misaligned gate or
 * workspace, a workspace below the size above, a misaligned norm_w, a bad eps,
 * spin_limit < -1 or overlapping buffers.
 */
int kda_chunk_fwd_gated(const void *q, const void *k, const void *v, const void *g,
                        const void *beta, const float *S0, const void *gate,
                        const float *norm_w, float eps, void *y, float *S_T,
                        void *workspace, size_t workspace_bytes,
                        int B, int T, int H, int dk, int dv, int dtype,
                        const kda_fwd_options *opts, void *stream);

/* Bytes of workspace kda_chunk_fwd_gated needs for these sizes (0 for invalid sizes). */
size_t kda_chunk_fwd_gated_workspace_size(int B, int H, int dv);

/*
 * kda_chunk_bwd -- backward pass of one KDA layer's recurrence (training).
 *
 * Defines (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读",
 * section 3.3: training runs the chunked form of the section 3.1 recurrence;
 * the pages derive no backward pass): the exact gradients of
 *     Loss = <dO, o> + <dS_T, S_T>
 * through kda_chunk_fwd's map (q, k, v, g, beta, S0) -> (o, S_T), i.e. the
 * reverse mode of the chunked recurrence with 16-token chunks.  The call first
 * recomputes every chunk's incoming state (a forward pass into the workspace),
 * then walks the chunks from last to first.
 *
 *   q, k, g, v, beta, S0 : as kda_chunk_fwd (S0 NULL = zero initial state)
 *   dO    : [B, T, H, dv] (dtype)   upstream gradient of o
 *   dS_T  : [B, H, dk, dv] fp32     upstream gradient of S_T; NULL = zero
 *   dq, dk, dg : [B, T, H, dk] fp32 written
 *   dv    : [B, T, H, dv] fp32      written
 *   dbeta : [B, T, H] fp32          written
 *   dS0   : [B, H, dk, dv] fp32     written; NULL = not returned
 *   workspace : device memory of kda_chunk_bwd_workspace_size(B, T, H, dk, dv)
 *               bytes (may be NULL when that size is 0, i.e. T = 0), 256-byte
 *               aligned; its contents on entry are ignored and on return
 *               unspecified.  It holds every chunk's incoming state (sized as
 *               fp32 for either dtype) and, for dv = 128, the first value
 *               slice's partial dq, dk, dg, dbeta and two counters per (sequence,
 *               head): one through which the second slice's workgroup learns
 *               that they are complete, one that paces the first slice
 *   dk, dv (sizes) : 64 or 128
 * Gradients are fp32 in both dtype modes.  No output may overlap an input or
 * another output.  With dv = 128 the two value slices of a head hand partial
 * sums to each other through an XCD's L2; should the second find the first on
 * another XCD, or wait for it past the built-in limit, all of that head's dq,
 * dk, dg and dbeta are NaN (dv, dS0 stay exact).
 * Errors: KDA_ERR_INVALID (null/misaligned pointer, bad size, workspace too
 * small, overlap), KDA_ERR_UNSUPPORTED, KDA_ERR_LAUNCH.
 */
int kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g,
                  const void *beta, const float *S0, const void *dO, const float *dS_T,
                  float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                  void *workspace, size_t workspace_bytes,
                  int B, int T, int H, int dk_size, int dv_size, int dtype, void *stream);

/*
 * kda_chunk_bwd_ex -- kda_chunk_bwd with options, for testing the failure
 * marking of the two value slices' hand-off (dv = 128).
 *   opts : NULL = kda_chunk_bwd; else fail_xcd_check != 0 makes the second
 *          slice of every head take the first for one on another XCD, so that
 *          all of the head's dq, dk, dg and dbeta come out NaN while dv and dS0
 *          stay exact (the path a real mismatch or a wait that gave up takes).
 * Errors: as kda_chunk_bwd.
 */
typedef struct kda_bwd_options {
    int fail_xcd_check;
} kda_bwd_options;

int kda_chunk_bwd_ex(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, const float *S0, const void *dO, const float *dS_T,
                     float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                     void *workspace, size_t workspace_bytes,
                     int B, int T, int H, int dk_size, int dv_size, int dtype,
                     const kda_bwd_options *opts, void *stream);

/* Bytes of workspace kda_chunk_bwd needs for these sizes (0 for invalid sizes). */
size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int dk_size, int dv_size);

/*
 * kda_chunk_bwd_noalloc -- kda_chunk_bwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight training loops, harnesses
 * that forbid hipMalloc): the same kernels and results, with the workspace
 * taken from a device array the library holds instead of a caller's buffer.
 *
 *   Arguments, layouts and gradients as kda_chunk_bwd, without the workspace
 *   arguments.  The call allocates nothing and frees nothing.
 *   Scratch: a static device array of KDA_NOALLOC_SCRATCH_BYTES (64 MiB) in
 *     every GPU's memory, reserved when the library's code is loaded on that
 *     GPU and held until the process ends; its address is looked up once per
 *     device, on the first call with that device current.  Sizes whose
 *     kda_chunk_bwd_workspace_size exceeds it are rejected with
 *     KDA_ERR_TOO_LARGE (at dk = dv = 128 up to about 11900 token-heads,
 *     B*H*T, fit).  The array's contents on entry are ignored.
 *   Concurrency: every call on one GPU uses that GPU's single array, so calls
 *     whose work can overlap on one GPU (different streams, or different
 *     host threads, without ordering between them) race and give wrong
 *     gradients; calls ordered on one stream are safe.
 *   stream: must belong to the current device (KDA_ERR_INVALID otherwise).
 * Errors: as kda_chunk_bwd, plus KDA_ERR_TOO_LARGE.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int kda_chunk_bwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                          const void *beta, const float *S0, const void *dO, const float *dS_T,
                          float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                          int B, int T, int H, int dk_size, int dv_size, int dtype, void *stream);

/*
 * kda_validate_inputs -- debug check of the value domains the kernels assume
 * (the "values outside the stated domains" of the conventions above).
 *
 * Domains (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读",
 * section 3.3, lower-bounded decay: g in [g_min, 0], g_min = -5; section 3.1:
 * beta in [0, 1], the write strength of the delta rule).  NaN is outside both.
 *
 *   g      : [B, T, H, dk] (dtype)   as passed to kda_chunk_fwd
 *   beta   : [B, T, H]     (dtype)
 *   report : DEVICE int64[4], 8-byte aligned, written:
 *            report[0] = number of g elements outside [-5, 0]
 *            report[1] = flat index of the first of them, -1 if none
 *            report[2], report[3] = the same for beta outside [0, 1]
 * Enqueued on `stream` like every other entry point (read the report after the
 * stream has finished).  Errors: KDA_ERR_INVALID (null report or null tensor
 * with elements, bad size or dtype, misaligned report), KDA_ERR_LAUNCH.
 */
int kda_validate_inputs(const void *g, const void *beta, long long *report,
                        int B, int T, int H, int dk, int dtype, void *stream);

/* Human-readable text for a kda_status code (static storage, never NULL). */
const char *kda_strerror(int status);

/*
 * kda_workgroup_xcds -- debug check of the workgroup placement the fused
 * launches rely on.
 *
 * The launches whose workgroups hand data to each other through the L2
 * (kda_chunk_fwd_gated, kda_chunk_fwd_from_proj, and kda_chunk_bwd with dv = 128)
 * assume that a launch's workgroups go round-robin over the 8 XCDs (accelerator
 * dies), so that workgroups i and i + 8 -- a writer and its readers -- share a
 * die's L2; which XCD takes workgroup 0 varies between launches.  Each of them
 * checks the assumption at run time (hand-off words carry the writer's XCD) and
 * marks its outputs NaN where it fails.  This enqueues one launch
 * of n workgroups, each requesting lds_bytes of dynamic LDS (as those kernels
 * do), in which workgroup i writes the XCD it ran on to xcd[i].
 *   xcd       : device int32 [n], written
 *   n         : 0 .. 2^20 workgroups (0: nothing is enqueued)
 *   lds_bytes : 0 .. 163840
 * Errors: KDA_ERR_INVALID for sizes outside those ranges or a null or misaligned
 * xcd; KDA_ERR_LAUNCH if the runtime rejects the launch.
 */
int kda_workgroup_xcds(int *xcd, int n, int lds_bytes, void *stream);

/* KDA_VERSION of the loaded library. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
