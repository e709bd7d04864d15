/*
 * kda_oracle.c -- plain, slow fp64 reference of the Kimi Delta Attention (KDA)
 * layer recurrence, for testing only.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU path, and the GPU path never calls it.
 *
 * Sources (web pages; cited by title and section):
 *   [note]  "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读" (a reading note
 *           on the Kimi K3 report), section 3.1 "从“不断累加”到“按地址改写”" and
 *           section 3.2 "单个 token 的输入、状态与输出".
 *   [essay] "Kimi K3 架构篇：一文详解 2.8 万亿参数的巨型怪兽", section
 *           "KDA 到底在算什么：把公式摊开".
 *
 * What is computed, per (sequence, head), token by token, in the order the
 * note's section 3.2 gives for one step:
 *     alpha_t = exp(g_t)                      (per key channel; section 3.3 maps
 *                                              g into (g_min, 0) and alpha = exp g)
 *     Sbar    = Diag(alpha_t) S_{t-1}         (rows = key channels are scaled)
 *     vhat_t  = Sbar^T k_t                    (old prediction at address k_t)
 *     S_t     = Sbar + beta_t k_t (v_t - vhat_t)^T
 *     o_t     = S_t^T q_t                     (read after the write)
 * This equals the closed recurrence S_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
 * S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t of the note's section 3.1 and of
 * the essay.  No 1/sqrt(d_k) scale is applied to q (the pages apply none).
 *
 * The decode step additionally prepares q, k, v from their projected
 * pre-activations as the note's section 3.2 input-branch equation states:
 * q, k = L2Norm(Swish(ShortConv(x))), v = Swish(ShortConv(x)).  The pages do not
 * fix the conv width, its bias, Swish's parameter or L2Norm's epsilon; the
 * readings used here are: depthwise causal conv of width `width` without bias,
 * tap 0 applied to the oldest token; Swish(u) = u * sigmoid(u); L2Norm(x) =
 * x / sqrt(sum x^2 + eps).
 *
 * Prefill preprocessing applies the same input branches to a whole sequence of
 * projected pre-activations (the conv window reaching back into a caller-given
 * history of width-1 tokens before the first one) and adds the two scalar maps
 * of the note: beta_t = Sigmoid(beta logit) (section 3.2) and the lower-bounded
 * decay of section 3.3, g_t = g_min * Sigmoid(e^{A^h} z_t) with g_min = -5 and
 * A^h one number per head.
 *
 * Prefill can also record the state at regular token counts: the note's
 * section 9 (long-trajectory environments, the report's Figure 12 on prefix
 * caching) keeps one KDA state per sequence and layer and snapshots it only at
 * block boundaries (512 tokens), so that a cached prefix resumes prefill from
 * the state at its end.  Snapshot s is the state after the first
 * (s + 1) * snap_every tokens, i.e. exactly what a prefill over that prefix
 * returns as its final state.
 *
 * Layouts (all row-major, fp64, host memory):
 *   q, k, g : [B, T, H, dk]     v, o : [B, T, H, dv]     beta : [B, T, H]
 *   S0, S_T : [B, H, dk, dv]    (row = key channel, column = value channel)
 *   snaps   : [n_snaps, B, H, dk, dv]
 * Independent (b, h) units are spread over `nthreads` POSIX threads; each
 * unit's loop is sequential.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *S0;
    double *o, *S_T;
    double *snaps;
    long snap_every, n_snaps;
    long B, T, H, dk, dv;
    int tid, nthreads;
    int status;
} prefill_job;

/* One (b, h) unit: the token-serial loop of the note's section 3.2. */
static void prefill_unit(const prefill_job *J, long b, long h, double *S, double *vhat)
{
    const long dk = J->dk, dv = J->dv, H = J->H, T = J->T;
    if (J->S0)
        memcpy(S, J->S0 + (b * H + h) * dk * dv, sizeof(double) * dk * dv);
    else
        memset(S, 0, sizeof(double) * dk * dv);

    for (long t = 0; t < T; ++t) {
        const long tok = (b * T + t) * H + h;
        const double *qt = J->q + tok * dk;
        const double *kt = J->k + tok * dk;
        const double *gt = J->g + tok * dk;
        const double *vt = J->v + tok * dv;
        const double bt = J->beta[tok];
        double *ot = J->o + tok * dv;

        /* Sbar = Diag(exp(g_t)) S : scale row i by alpha_i */
        for (long i = 0; i < dk; ++i) {
            const double a = exp(gt[i]);
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] *= a;
        }
        /* vhat = Sbar^T k */
        for (long j = 0; j < dv; ++j)
            vhat[j] = 0.0;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                vhat[j] += S[i * dv + j] * kt[i];
        /* S = Sbar + beta k (v - vhat)^T */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] += bt * kt[i] * (vt[j] - vhat[j]);
        /* o = S^T q */
        for (long j = 0; j < dv; ++j)
            ot[j] = 0.0;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                ot[j] += S[i * dv + j] * qt[i];
        /* the state after t + 1 tokens, when that count closes a snapshot block */
        if (J->snaps && (t + 1) % J->snap_every == 0 && (t + 1) / J->snap_every <= J->n_snaps) {
            const long s = (t + 1) / J->snap_every - 1;
            memcpy(J->snaps + ((s * J->B + b) * H + h) * dk * dv, S, sizeof(double) * dk * dv);
        }
    }
    if (J->S_T)
        memcpy(J->S_T + (b * H + h) * dk * dv, S, sizeof(double) * dk * dv);
}

static void *prefill_worker(void *arg)
{
    prefill_job *J = (prefill_job *)arg;
    double *S = (double *)malloc(sizeof(double) * J->dk * J->dv);
    double *vhat = (double *)malloc(sizeof(double) * J->dv);
    if (!S || !vhat) {
        J->status = -1;
        free(S);
        free(vhat);
        return NULL;
    }
    for (long u = J->tid; u < J->B * J->H; u += J->nthreads)
        prefill_unit(J, u / J->H, u % J->H, S, vhat);
    free(S);
    free(vhat);
    return NULL;
}

/*
 * Prefill over T tokens for B sequences and H heads, recording n_snaps states
 * (snapshot s after (s + 1) * snap_every tokens; n_snaps * snap_every <= T).
 * S0 may be NULL (zero initial state); S_T may be NULL (final state not
 * returned); snaps may be NULL when n_snaps is 0.  S0 and S_T may alias.
 * Returns 0, or -1 on a bad argument or failed allocation.
 */
int kda_oracle_prefill_snapshots(const double *q, const double *k, const double *v,
                                 const double *g, const double *beta, const double *S0, double *o,
                                 double *S_T, double *snaps, long snap_every, long n_snaps,
                                 long B, long T, long H, long dk, long dv, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !o || B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -1;
    if (n_snaps < 0 || (n_snaps > 0 && (!snaps || snap_every <= 0 || n_snaps * snap_every > T)))
        return -1;
    if (n_snaps == 0)
        snaps = NULL;
    if (nthreads < 1)
        nthreads = 1;
    if ((long)nthreads > B * H)
        nthreads = (int)(B * H > 0 ? B * H : 1);

    prefill_job *jobs = (prefill_job *)calloc((size_t)nthreads, sizeof(prefill_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        prefill_job J = {q, k, v, g, beta, S0, o, S_T, snaps, snap_every, n_snaps, B, T, H, dk, dv, i, nthreads, 0};
        jobs[i] = J;
    }
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, prefill_worker, &jobs[i]) != 0)
            jobs[i].status = -2; /* run it inline below instead */
    prefill_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) {
        if (jobs[i].status == -2) {
            jobs[i].status = 0;
            prefill_worker(&jobs[i]);
        } else {
            pthread_join(th[i], NULL);
        }
    }
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status)
            rc = -1;
    free(jobs);
    free(th);
    return rc;
}

/* Prefill without snapshots (see above). */
int kda_oracle_prefill(const double *q, const double *k, const double *v, const double *g,
                       const double *beta, const double *S0, double *o, double *S_T,
                       long B, long T, long H, long dk, long dv, int nthreads)
{
    return kda_oracle_prefill_snapshots(q, k, v, g, beta, S0, o, S_T, NULL, 1, 0, B, T, H, dk, dv,
                                        nthreads);
}

/* ---------------------------------------------------------------- decode -- */

typedef struct {
    const double *q_pre, *k_pre, *v_pre, *conv_w, *g, *beta;
    double *conv_cache, *S, *o;
    long conv_pos, N, H, dk, dv, width;
    double eps;
    int tid, nthreads;
    int status;
} decode_job;

static double swish(double u) { return u / (1.0 + exp(-u)); }

static void decode_unit(const decode_job *J, long n, long h, double *x, double *act,
                        double *vhat)
{
    const long dk = J->dk, dv = J->dv, H = J->H, W = J->width;
    const long nch = 2 * dk + dv;           /* channels: q | k | v */
    const long nh = n * H + h;
    double *cache = J->conv_cache + nh * (W - 1) * nch;
    const double *w = J->conv_w + h * nch * W;
    const long oldest = J->conv_pos % (W - 1);

    /* the current token's projected pre-activations, channel order q|k|v */
    for (long c = 0; c < dk; ++c) x[c] = J->q_pre[nh * dk + c];
    for (long c = 0; c < dk; ++c) x[dk + c] = J->k_pre[nh * dk + c];
    for (long c = 0; c < dv; ++c) x[2 * dk + c] = J->v_pre[nh * dv + c];

    /* ShortConv: window = (W-1 cached tokens, oldest first) followed by x_t */
    for (long c = 0; c < nch; ++c) {
        double u = 0.0;
        for (long j = 0; j < W - 1; ++j) {
            const long slot = (oldest + j) % (W - 1);
            u += w[c * W + j] * cache[slot * nch + c];
        }
        u += w[c * W + (W - 1)] * x[c];
        act[c] = swish(u);
    }
    /* the cache forgets its oldest token and keeps x_t in that slot */
    for (long c = 0; c < nch; ++c)
        cache[oldest * nch + c] = x[c];

    /* L2Norm on q and on k */
    double sq = 0.0, sk = 0.0;
    for (long c = 0; c < dk; ++c) {
        sq += act[c] * act[c];
        sk += act[dk + c] * act[dk + c];
    }
    const double rq = 1.0 / sqrt(sq + J->eps), rk = 1.0 / sqrt(sk + J->eps);
    for (long c = 0; c < dk; ++c) {
        act[c] *= rq;
        act[dk + c] *= rk;
    }
    const double *qt = act, *kt = act + dk, *vt = act + 2 * dk;
    const double *gt = J->g + nh * dk;
    const double bt = J->beta[nh];
    double *S = J->S + nh * dk * dv;
    double *ot = J->o + nh * dv;

    /* the single-token state edit, same order as the prefill loop */
    for (long i = 0; i < dk; ++i) {
        const double a = exp(gt[i]);
        for (long j = 0; j < dv; ++j)
            S[i * dv + j] *= a;
    }
    for (long j = 0; j < dv; ++j)
        vhat[j] = 0.0;
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j)
            vhat[j] += S[i * dv + j] * kt[i];
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j)
            S[i * dv + j] += bt * kt[i] * (vt[j] - vhat[j]);
    for (long j = 0; j < dv; ++j)
        ot[j] = 0.0;
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j)
            ot[j] += S[i * dv + j] * qt[i];
}

static void *decode_worker(void *arg)
{
    decode_job *J = (decode_job *)arg;
    const long nch = 2 * J->dk + J->dv;
    double *x = (double *)malloc(sizeof(double) * nch);
    double *act = (double *)malloc(sizeof(double) * nch);
    double *vhat = (double *)malloc(sizeof(double) * J->dv);
    if (!x || !act || !vhat) {
        J->status = -1;
    } else {
        for (long u = J->tid; u < J->N * J->H; u += J->nthreads)
            decode_unit(J, u / J->H, u % J->H, x, act, vhat);
    }
    free(x);
    free(act);
    free(vhat);
    return NULL;
}

/*
 * One decode step for N sequences and H heads.
 *   q_pre, k_pre [N,H,dk], v_pre [N,H,dv]: projected pre-activations of x_t
 *   conv_w [H, 2dk+dv, width]: depthwise taps, tap 0 = oldest token
 *   conv_cache [N,H,width-1, 2dk+dv]: ring of the previous width-1 tokens;
 *       slot (conv_pos mod (width-1)) holds the oldest and is overwritten with x_t
 *   g [N,H,dk], beta [N,H]; S [N,H,dk,dv] updated in place; o [N,H,dv]
 * Returns 0, or -1 on a bad argument or failed allocation.
 */
int kda_oracle_decode_step(const double *q_pre, const double *k_pre, const double *v_pre,
                           const double *conv_w, double *conv_cache, long conv_pos,
                           const double *g, const double *beta, double *S, double *o,
                           long N, long H, long dk, long dv, long width, double eps,
                           int nthreads)
{
    if (!q_pre || !k_pre || !v_pre || !conv_w || !conv_cache || !g || !beta || !S || !o ||
        N < 0 || H < 0 || dk <= 0 || dv <= 0 || width < 2 || conv_pos < 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if ((long)nthreads > N * H)
        nthreads = (int)(N * H > 0 ? N * H : 1);
    decode_job *jobs = (decode_job *)calloc((size_t)nthreads, sizeof(decode_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        decode_job J = {q_pre, k_pre, v_pre, conv_w, g, beta, conv_cache, S, o,
                        conv_pos, N, H, dk, dv, width, eps, i, nthreads, 0};
        jobs[i] = J;
    }
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, decode_worker, &jobs[i]) != 0)
            jobs[i].status = -2;
    decode_worker(&jobs[0]);
    int rc = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (jobs[i].status == -2) {
            jobs[i].status = 0;
            decode_worker(&jobs[i]);
        } else {
            pthread_join(th[i], NULL);
        }
    }
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status)
            rc = -1;
    free(jobs);
    free(th);
    return rc;
}

/* ------------------------------------------------------ prefill preprocessing -- */

typedef struct {
    const double *q_pre, *k_pre, *v_pre, *conv_w, *conv_init, *z, *A, *beta_logit;
    double *q, *k, *v, *g, *beta, *conv_final;
    long B, T, H, dk, dv, width;
    double eps;
    int tid, nthreads;
} prep_job;

static double sigmoid(double u) { return 1.0 / (1.0 + exp(-u)); }

/* Pre-activation of channel c (order q | k | v) at token t of unit (b, h); t < 0
 * reaches into the history: conv_init[b, h, (width-1) + t, c], or 0 without one. */
static double pre_at(const prep_job *J, long b, long h, long t, long c)
{
    const long dk = J->dk, dv = J->dv, H = J->H, nch = 2 * dk + dv;
    if (t < 0) {
        if (!J->conv_init)
            return 0.0;
        return J->conv_init[((b * H + h) * (J->width - 1) + (J->width - 1) + t) * nch + c];
    }
    const long tok = (b * J->T + t) * H + h;
    if (c < dk)
        return J->q_pre[tok * dk + c];
    if (c < 2 * dk)
        return J->k_pre[tok * dk + c - dk];
    return J->v_pre[tok * dv + c - 2 * dk];
}

/* One (b, h) unit, token by token (note, sections 3.2 and 3.3). */
static void prep_unit(const prep_job *J, long b, long h, double *act)
{
    const long dk = J->dk, dv = J->dv, H = J->H, W = J->width, nch = 2 * dk + dv;
    const double *w = J->conv_w + h * nch * W;
    const double eA = exp(J->A[h]);
    for (long t = 0; t < J->T; ++t) {
        const long tok = (b * J->T + t) * H + h;
        /* ShortConv over the window t-W+1 .. t (tap 0 = oldest), then Swish */
        for (long c = 0; c < nch; ++c) {
            double u = 0.0;
            for (long j = 0; j < W; ++j)
                u += w[c * W + j] * pre_at(J, b, h, t - (W - 1) + j, c);
            act[c] = swish(u);
        }
        /* L2Norm of the q part and of the k part */
        double sq = 0.0, sk = 0.0;
        for (long c = 0; c < dk; ++c) {
            sq += act[c] * act[c];
            sk += act[dk + c] * act[dk + c];
        }
        const double rq = 1.0 / sqrt(sq + J->eps), rk = 1.0 / sqrt(sk + J->eps);
        for (long c = 0; c < dk; ++c) {
            J->q[tok * dk + c] = act[c] * rq;
            J->k[tok * dk + c] = act[dk + c] * rk;
        }
        for (long c = 0; c < dv; ++c)
            J->v[tok * dv + c] = act[2 * dk + c];
        /* the two scalar maps */
        J->beta[tok] = sigmoid(J->beta_logit[tok]);
        for (long c = 0; c < dk; ++c)
            J->g[tok * dk + c] = -5.0 * sigmoid(eA * J->z[tok * dk + c]);
    }
    /* the history the next call continues from: the last width-1 pre-activations */
    if (J->conv_final)
        for (long j = 0; j < W - 1; ++j)
            for (long c = 0; c < nch; ++c)
                J->conv_final[((b * H + h) * (W - 1) + j) * nch + c] =
                    pre_at(J, b, h, J->T - (W - 1) + j, c);
}

static void *prep_worker(void *arg)
{
    prep_job *J = (prep_job *)arg;
    double *act = (double *)malloc(sizeof(double) * (size_t)(2 * J->dk + J->dv));
    if (act)
        for (long u = J->tid; u < J->B * J->H; u += J->nthreads)
            prep_unit(J, u / J->H, u % J->H, act);
    free(act);
    return act ? NULL : (void *)1;
}

/*
 * Prefill preprocessing of B sequences of T tokens and H heads.
 *   q_pre, k_pre, z [B,T,H,dk]; v_pre [B,T,H,dv]; beta_logit [B,T,H]
 *   conv_w [H, 2dk+dv, width] (tap 0 = oldest); A [H]
 *   conv_init [B,H,width-1,2dk+dv] oldest first, or NULL for a zero history
 * Writes q, k, g [B,T,H,dk], v [B,T,H,dv], beta [B,T,H] and, when conv_final is
 * not NULL, conv_final [B,H,width-1,2dk+dv]: the last width-1 pre-activations,
 * oldest first (reaching into conv_init when T < width-1).  conv_final must not
 * overlap conv_init.  Returns 0, or -1 on a bad argument or failed allocation.
 */
int kda_oracle_prefill_prep(const double *q_pre, const double *k_pre, const double *v_pre,
                            const double *conv_w, const double *conv_init, const double *z,
                            const double *A, const double *beta_logit,
                            double *q, double *k, double *v, double *g, double *beta,
                            double *conv_final, long B, long T, long H, long dk, long dv,
                            long width, double eps, int nthreads)
{
    if (!q_pre || !k_pre || !v_pre || !conv_w || !z || !A || !beta_logit || !q || !k || !v ||
        !g || !beta || B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || width < 2)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if ((long)nthreads > B * H)
        nthreads = (int)(B * H > 0 ? B * H : 1);
    prep_job *jobs = (prep_job *)calloc((size_t)nthreads, sizeof(prep_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        prep_job J = {q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit,
                      q, k, v, g, beta, conv_final, B, T, H, dk, dv, width, eps, i, nthreads};
        jobs[i] = J;
    }
    /* a worker whose thread could not start runs on the calling thread */
    char *started = (char *)calloc((size_t)nthreads, 1);
    if (started)
        for (int i = 1; i < nthreads; ++i)
            started[i] = pthread_create(&th[i], NULL, prep_worker, &jobs[i]) == 0;
    if (prep_worker(&jobs[0]))
        rc = -1;
    for (int i = 1; i < nthreads; ++i) {
        void *ret = NULL;
        if (started && started[i])
            pthread_join(th[i], &ret);
        else
            ret = prep_worker(&jobs[i]);
        if (ret)
            rc = -1;
    }
    free(started);
    free(jobs);
    free(th);
    return rc;
}

/*
 * Output exposure gate (note, section 3.2, output equation
 * y_t = W_o[Sigmoid(W_g x_t) (.) RMSNorm(o~_t)], without the W_o projection,
 * which needs trained weights).  The note says RMSNorm steadies each head's
 * readout, so it normalises the dv channels of one (token, head):
 *     y[r,h,c] = Sigmoid(gate[r,h,c]) * o[r,h,c] / sqrt(mean_c' o[r,h,c']^2 + eps) * w[c]
 * Readings where the pages are silent: RMSNorm carries a per-channel weight w
 * (NULL = all ones) shared by the heads, and eps is the caller's.
 *   o, gate, y : [rows, H, dv]     w : [dv] or NULL
 * Returns 0, or -1 on a bad argument.
 */
int kda_oracle_output_gate(const double *o, const double *gate, const double *w, double *y,
                           long rows, long H, long dv, double eps)
{
    if (!o || !gate || !y || rows < 0 || H < 0 || dv <= 0 || !(eps >= 0.0))
        return -1;
    for (long u = 0; u < rows * H; ++u) {
        const double *ou = o + u * dv, *gu = gate + u * dv;
        double ss = 0.0;
        for (long c = 0; c < dv; ++c)
            ss += ou[c] * ou[c];
        const double inv_rms = 1.0 / sqrt(ss / (double)dv + eps);
        for (long c = 0; c < dv; ++c)
            y[u * dv + c] = sigmoid(gu[c]) * ou[c] * inv_rms * (w ? w[c] : 1.0);
    }
    return 0;
}
