/*
 * kda_oracle.c -- plain fp64 token-by-token recurrence of the KDA scan.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the correctness oracle that the HIP
 * path is checked against. Only the tests, the smoke check and the CPU
 * baseline of the benchmark may load it; the product path never does. It
 * shares no code, header or table with the HIP library.
 *
 * What it computes (Chimera, arXiv 2607.28611):
 *   - the state update printed in the explainer page, section "One stream,
 *     three mechanisms, no positions":
 *         S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     with alpha_t in (0,1)^{d_k} a per-key-channel forget gate and beta_t a
 *     scalar write/erase strength (paper Sec. 3, KDA paragraph, Eq. 14);
 *   - S_t in R^{d_k x d_v} is the state after processing position t, and the
 *     state is reset to S_0 = 0 at every packed-sample boundary (same paragraph);
 *   - every head uses the same causal scan order (same paragraph);
 *   - readout o_t = S_t^T q_t from the post-update state. The display
 *     equation that states the readout did not survive extraction; this is
 *     the plain reading of the definitions (S_t is the state "after
 *     processing" position t, q_t in R^{d_q} with d_q = d_k, no scale). The
 *     pages themselves print no readout, so its form is a reading; the
 *     exact-recall pin fixes that it uses the post-update state.
 *
 * The update is evaluated in its expanded form, token by token:
 *     S~ = Diag(alpha) S            decay each key row
 *     p  = S~^T k                   what the decayed state returns for k
 *     u  = beta (v - p)             innovation
 *     S  = S~ + k u^T               (I - beta k k^T) S~ + beta k v^T
 *     o  = S^T q
 * All arithmetic is fp64 with libm exp; inputs arrive as fp64 (exact upcasts
 * of the stored fp32/bf16 values). There is no chunking, blocking or reordering.
 *
 * Layout: q, k, log_alpha [T][H][dk]; v, out [T][H][dv]; beta [T][H];
 * cu_seqlens int32 [N+1]; final_state [N][H][dk][dv] (rows = key channels).
 *
 * kda_oracle_forward_from additionally takes initial_state [N][H][dk][dv]: the
 * state a sample starts from in place of 0, for continuing a scan from a retained
 * state (the per-head state is all a sample carries forward: explainer page "What
 * O(N) buys in memory and latency"; paper Sec. 5 efficiency study, Fig. 18,
 * roll-out-cache setting). Everything else is the same recurrence.
 *
 * kda_oracle_forward_ex also takes qk_l2norm: when nonzero, q_t and k_t of every
 * (token, head) are first divided by their Euclidean length (a zero vector stays
 * zero) and the recurrence then runs on the unit vectors. The paper's training
 * setup names chunked KDA kernels with fused normalization; its form is not
 * printed. The form taken is the per-token L2 normalisation of queries and keys:
 * with a unit key, I - beta k k^T scales the state's component along k by 1 - beta,
 * so that beta acts as the erase fraction the paper's KDA paragraph describes.
 *
 * kda_oracle_backward is the reverse-mode derivative of the same recurrence (the
 * paper trains with these kernels: training setup paragraph on the custom kernels).
 * For a scalar loss L with dL/do_t = d_out[t] and dL/dS_final = d_final_state it
 * returns dL/dq, dL/dk, dL/dv, dL/dlog_alpha, dL/dbeta and dL/dS_0, walking the
 * tokens of each (sample, head) backwards and applying the chain rule to the
 * expanded update above, one step at a time:
 *     dS   += q do^T                      o = S^T q
 *     dq    = S do
 *     du    = dS^T k,   dk = dS u         S = S~ + k u^T
 *     dbeta = du.(v - p),  dv = beta du,  dp = -beta du
 *     dS~   = dS + k dp^T,  dk += S~ dp   p = S~^T k
 *     dlog_alpha_c = sum_j dS~[c][j] S~[c][j],  dS_prev = Diag(alpha) dS~
 * and, with qk_l2norm, dx = (dx^ - x^ (x^ . dx^)) / |x| for x^ = x / |x| (0 for x = 0).
 * The states S_{t-1} the reverse walk needs are replayed forward from the state
 * kept every 64 tokens: the same fp64 operations in the same order, so the replayed
 * values are the forward values bit for bit.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *log_alpha, *beta;
    const int32_t *cu_seqlens;
    const double *initial_state;   /* NULL = S_0 = 0 */
    int32_t qk_l2norm;             /* nonzero: unit-length q_t, k_t */
    int32_t n_seqs, H, dk, dv;
    const uint8_t *head_mask;   /* NULL = all heads */
    double *out, *final_state;
    /* work queue over (sequence, head) units */
    pthread_mutex_t lock;
    int64_t next_unit;
    int failed;
} oracle_job;

/* One (sequence, head) unit: the recurrence over the tokens of that sample. */
static int scan_unit(oracle_job *job, int32_t n, int32_t h)
{
    const int32_t H = job->H, dk = job->dk, dv = job->dv;
    const int64_t t0 = job->cu_seqlens[n], t1 = job->cu_seqlens[n + 1];
    double *S = calloc((size_t)dk * dv, sizeof(double));   /* reset: S_0 = 0 */
    double *p = malloc(sizeof(double) * dv);
    double *u = malloc(sizeof(double) * dv);
    double *qn = malloc(sizeof(double) * dk);
    double *kn = malloc(sizeof(double) * dk);
    if (!S || !p || !u || !qn || !kn) { free(S); free(p); free(u); free(qn); free(kn); return -1; }
    if (job->initial_state)
        memcpy(S, job->initial_state + ((size_t)n * H + h) * dk * dv, sizeof(double) * dk * dv);

    for (int64_t t = t0; t < t1; ++t) {
        const double *kt = job->k + (t * H + h) * dk;
        const double *qt = job->q + (t * H + h) * dk;
        if (job->qk_l2norm) {
            /* q_t / |q_t|, k_t / |k_t| (a zero vector stays zero) */
            double sq = 0.0, sk = 0.0;
            for (int32_t c = 0; c < dk; ++c) { sq += qt[c] * qt[c]; sk += kt[c] * kt[c]; }
            sq = sq > 0.0 ? 1.0 / sqrt(sq) : 0.0;
            sk = sk > 0.0 ? 1.0 / sqrt(sk) : 0.0;
            for (int32_t c = 0; c < dk; ++c) { qn[c] = qt[c] * sq; kn[c] = kt[c] * sk; }
            qt = qn;
            kt = kn;
        }
        const double *lat = job->log_alpha + (t * H + h) * dk;
        const double *vt = job->v + (t * H + h) * dv;
        const double bt = job->beta[t * H + h];

        /* decay: S~ = Diag(alpha_t) S_{t-1}, alpha = exp(log alpha) per key channel */
        for (int32_t c = 0; c < dk; ++c) {
            const double a = exp(lat[c]);
            double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) row[j] *= a;
        }
        /* p = S~^T k_t */
        for (int32_t j = 0; j < dv; ++j) p[j] = 0.0;
        for (int32_t c = 0; c < dk; ++c) {
            const double kc = kt[c];
            const double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) p[j] += row[j] * kc;
        }
        /* u = beta_t (v_t - p) */
        for (int32_t j = 0; j < dv; ++j) u[j] = bt * (vt[j] - p[j]);
        /* S_t = S~ + k_t u^T */
        for (int32_t c = 0; c < dk; ++c) {
            const double kc = kt[c];
            double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) row[j] += kc * u[j];
        }
        /* o_t = S_t^T q_t */
        double *ot = job->out + (t * H + h) * dv;
        for (int32_t j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int32_t c = 0; c < dk; ++c) {
            const double qc = qt[c];
            const double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) ot[j] += row[j] * qc;
        }
    }
    if (job->final_state)
        memcpy(job->final_state + ((size_t)n * H + h) * dk * dv, S, sizeof(double) * dk * dv);
    free(S); free(p); free(u); free(qn); free(kn);
    return 0;
}

static void *worker(void *arg)
{
    oracle_job *job = (oracle_job *)arg;
    const int64_t units = (int64_t)job->n_seqs * job->H;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        const int64_t i = job->next_unit++;
        pthread_mutex_unlock(&job->lock);
        if (i >= units) break;
        const int32_t n = (int32_t)(i / job->H), h = (int32_t)(i % job->H);
        if (job->head_mask && !job->head_mask[h]) continue;
        if (scan_unit(job, n, h) != 0) {
            pthread_mutex_lock(&job->lock);
            job->failed = 1;
            pthread_mutex_unlock(&job->lock);
        }
    }
    return NULL;
}

/*
 * Run the recurrence for every (sequence, head) unit, or for the heads whose
 * head_mask entry is nonzero. out rows of skipped heads are left untouched.
 * initial_state NULL means every sample starts from 0. threads <= 0 means one
 * thread. Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int kda_oracle_forward_ex(const double *q, const double *k, const double *v,
                          const double *log_alpha, const double *beta,
                          const int32_t *cu_seqlens, const double *initial_state, int32_t qk_l2norm,
                          int32_t n_seqs, int32_t H, int32_t dk, int32_t dv,
                          const uint8_t *head_mask, double *out, double *final_state,
                          int32_t threads)
{
    if (!cu_seqlens || n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (cu_seqlens[0] != 0) return -1;
    for (int32_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !log_alpha || !beta || !out)) return -1;

    oracle_job job;
    memset(&job, 0, sizeof job);
    job.q = q; job.k = k; job.v = v; job.log_alpha = log_alpha; job.beta = beta;
    job.cu_seqlens = cu_seqlens; job.n_seqs = n_seqs; job.H = H; job.dk = dk; job.dv = dv;
    job.head_mask = head_mask; job.out = out; job.final_state = final_state;
    job.initial_state = initial_state;
    job.qk_l2norm = qk_l2norm;
    pthread_mutex_init(&job.lock, NULL);

    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int i = 1; i < threads; ++i)
        if (pthread_create(&tid[started], NULL, worker, &job) == 0) ++started;
    worker(&job);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    pthread_mutex_destroy(&job.lock);
    return job.failed ? -1 : 0;
}

/* The scan from given initial states, q and k used as stored. */
int kda_oracle_forward_from(const double *q, const double *k, const double *v,
                            const double *log_alpha, const double *beta,
                            const int32_t *cu_seqlens, const double *initial_state,
                            int32_t n_seqs, int32_t H, int32_t dk, int32_t dv,
                            const uint8_t *head_mask, double *out, double *final_state,
                            int32_t threads)
{
    return kda_oracle_forward_ex(q, k, v, log_alpha, beta, cu_seqlens, initial_state, 0, n_seqs, H,
                                 dk, dv, head_mask, out, final_state, threads);
}

/* The scan from zero states. */
int kda_oracle_forward(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta,
                       const int32_t *cu_seqlens, int32_t n_seqs, int32_t H,
                       int32_t dk, int32_t dv, const uint8_t *head_mask,
                       double *out, double *final_state, int32_t threads)
{
    return kda_oracle_forward_from(q, k, v, log_alpha, beta, cu_seqlens, NULL, n_seqs, H, dk, dv,
                                   head_mask, out, final_state, threads);
}

/* ------------------------------------------------------------------------- */
/* reverse mode                                                               */
/* ------------------------------------------------------------------------- */
#define KDA_ORACLE_REPLAY 64

typedef struct {
    const double *q, *k, *v, *log_alpha, *beta, *d_out, *d_final_state, *initial_state;
    const int32_t *cu_seqlens;
    int32_t qk_l2norm, n_seqs, H, dk, dv;
    double *dq, *dkey, *dval, *dlog_alpha, *dbeta, *d_initial_state;
    pthread_mutex_t lock;
    int64_t next_unit;
    int failed;
} oracle_bwd_job;

/* q_t or k_t as the recurrence uses it: x, or x / |x| with inv = 1/|x| (0 for x = 0) */
static void used_vector(const double *x, int32_t d, int norm, double *out, double *inv)
{
    if (!norm) {
        for (int32_t c = 0; c < d; ++c) out[c] = x[c];
        *inv = 1.0;
        return;
    }
    double s = 0.0;
    for (int32_t c = 0; c < d; ++c) s += x[c] * x[c];
    *inv = s > 0.0 ? 1.0 / sqrt(s) : 0.0;
    for (int32_t c = 0; c < d; ++c) out[c] = x[c] * *inv;
}

/* one forward token step S <- (I - beta k k^T) Diag(alpha) S + beta k v^T, keeping
   the decayed state S~ in St and p = S~^T k, u = beta (v - p) */
static void step_forward(double *S, double *St, double *p, double *u, const double *kt,
                         const double *lat, const double *vt, double bt, int32_t dk, int32_t dv)
{
    for (int32_t c = 0; c < dk; ++c) {
        const double a = exp(lat[c]);
        for (int32_t j = 0; j < dv; ++j) St[(size_t)c * dv + j] = S[(size_t)c * dv + j] * a;
    }
    for (int32_t j = 0; j < dv; ++j) p[j] = 0.0;
    for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j) p[j] += St[(size_t)c * dv + j] * kt[c];
    for (int32_t j = 0; j < dv; ++j) u[j] = bt * (vt[j] - p[j]);
    for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j) S[(size_t)c * dv + j] = St[(size_t)c * dv + j] + kt[c] * u[j];
}

static int backward_unit(oracle_bwd_job *job, int32_t n, int32_t h)
{
    const int32_t H = job->H, dk = job->dk, dv = job->dv, B = KDA_ORACLE_REPLAY;
    const int64_t t0 = job->cu_seqlens[n], t1 = job->cu_seqlens[n + 1], L = t1 - t0;
    const int64_t nblk = (L + B - 1) / B;
    const size_t SS = (size_t)dk * dv;
    double *ckpt = malloc(sizeof(double) * SS * (size_t)(nblk + 1));
    double *prev = malloc(sizeof(double) * SS * (size_t)B);     /* S_{t-1} of a block's tokens */
    double *S = malloc(sizeof(double) * SS), *St = malloc(sizeof(double) * SS);
    double *dS = malloc(sizeof(double) * SS), *dSt = malloc(sizeof(double) * SS);
    double *p = malloc(sizeof(double) * dv), *u = malloc(sizeof(double) * dv);
    double *du = malloc(sizeof(double) * dv), *dp = malloc(sizeof(double) * dv);
    double *qn = malloc(sizeof(double) * dk), *kn = malloc(sizeof(double) * dk);
    double *dqn = malloc(sizeof(double) * dk), *dkn = malloc(sizeof(double) * dk);
    int rc = 0;
    if (!ckpt || !prev || !S || !St || !dS || !dSt || !p || !u || !du || !dp || !qn || !kn || !dqn || !dkn) {
        rc = -1;
        goto done;
    }
    /* forward, keeping the state at the start of every block */
    if (job->initial_state) memcpy(S, job->initial_state + ((size_t)n * H + h) * SS, sizeof(double) * SS);
    else memset(S, 0, sizeof(double) * SS);
    for (int64_t t = t0; t < t1; ++t) {
        if ((t - t0) % B == 0) memcpy(ckpt + (size_t)((t - t0) / B) * SS, S, sizeof(double) * SS);
        double inv;
        used_vector(job->k + (t * H + h) * dk, dk, job->qk_l2norm, kn, &inv);
        step_forward(S, St, p, u, kn, job->log_alpha + (t * H + h) * dk, job->v + (t * H + h) * dv,
                     job->beta[t * H + h], dk, dv);
    }
    /* dL/dS_final */
    if (job->d_final_state) memcpy(dS, job->d_final_state + ((size_t)n * H + h) * SS, sizeof(double) * SS);
    else memset(dS, 0, sizeof(double) * SS);

    for (int64_t b = nblk - 1; b >= 0; --b) {
        const int64_t b0 = t0 + b * B, b1 = (b0 + B < t1) ? b0 + B : t1;
        /* replay the block forward from its kept state, recording S_{t-1} */
        memcpy(S, ckpt + (size_t)b * SS, sizeof(double) * SS);
        for (int64_t t = b0; t < b1; ++t) {
            memcpy(prev + (size_t)(t - b0) * SS, S, sizeof(double) * SS);
            double inv;
            used_vector(job->k + (t * H + h) * dk, dk, job->qk_l2norm, kn, &inv);
            step_forward(S, St, p, u, kn, job->log_alpha + (t * H + h) * dk, job->v + (t * H + h) * dv,
                         job->beta[t * H + h], dk, dv);
        }
        /* reverse walk over the block */
        for (int64_t t = b1 - 1; t >= b0; --t) {
            const double *lat = job->log_alpha + (t * H + h) * dk;
            const double *vt = job->v + (t * H + h) * dv;
            const double *dot = job->d_out + (t * H + h) * dv;
            const double bt = job->beta[t * H + h];
            double qinv, kinv;
            used_vector(job->q + (t * H + h) * dk, dk, job->qk_l2norm, qn, &qinv);
            used_vector(job->k + (t * H + h) * dk, dk, job->qk_l2norm, kn, &kinv);
            /* recompute step t from S_{t-1}: S~, p, u and S_t */
            memcpy(S, prev + (size_t)(t - b0) * SS, sizeof(double) * SS);
            step_forward(S, St, p, u, kn, lat, vt, bt, dk, dv);
            /* o_t = S_t^T q: dS += q do^T, dq = S_t do */
            for (int32_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) {
                    dS[(size_t)c * dv + j] += qn[c] * dot[j];
                    acc += S[(size_t)c * dv + j] * dot[j];
                }
                dqn[c] = acc;
            }
            /* S_t = S~ + k u^T: du = dS^T k, dk = dS u, dS~ = dS */
            for (int32_t j = 0; j < dv; ++j) du[j] = 0.0;
            for (int32_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) {
                    du[j] += dS[(size_t)c * dv + j] * kn[c];
                    acc += dS[(size_t)c * dv + j] * u[j];
                }
                dkn[c] = acc;
            }
            /* u = beta (v - p) */
            double db = 0.0;
            for (int32_t j = 0; j < dv; ++j) {
                db += du[j] * (vt[j] - p[j]);
                job->dval[(t * H + h) * dv + j] = bt * du[j];
                dp[j] = -bt * du[j];
            }
            job->dbeta[t * H + h] = db;
            /* p = S~^T k: dS~ = dS + k dp^T, dk += S~ dp */
            for (int32_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) {
                    dSt[(size_t)c * dv + j] = dS[(size_t)c * dv + j] + kn[c] * dp[j];
                    acc += St[(size_t)c * dv + j] * dp[j];
                }
                dkn[c] += acc;
            }
            /* S~ = Diag(alpha) S_{t-1}: dlog_alpha_c = sum_j dS~ S~, dS_{t-1} = Diag(alpha) dS~ */
            for (int32_t c = 0; c < dk; ++c) {
                const double a = exp(lat[c]);
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) {
                    acc += dSt[(size_t)c * dv + j] * St[(size_t)c * dv + j];
                    dS[(size_t)c * dv + j] = a * dSt[(size_t)c * dv + j];
                }
                job->dlog_alpha[(t * H + h) * dk + c] = acc;
            }
            /* through the normalisation x^ = x / |x|: dx = (dx^ - x^ (x^ . dx^)) / |x| */
            double *dqt = job->dq + (t * H + h) * dk, *dkt = job->dkey + (t * H + h) * dk;
            if (job->qk_l2norm) {
                double sq = 0.0, sk = 0.0;
                for (int32_t c = 0; c < dk; ++c) { sq += qn[c] * dqn[c]; sk += kn[c] * dkn[c]; }
                for (int32_t c = 0; c < dk; ++c) {
                    dqt[c] = (dqn[c] - qn[c] * sq) * qinv;
                    dkt[c] = (dkn[c] - kn[c] * sk) * kinv;
                }
            } else {
                for (int32_t c = 0; c < dk; ++c) { dqt[c] = dqn[c]; dkt[c] = dkn[c]; }
            }
        }
    }
    if (job->d_initial_state) memcpy(job->d_initial_state + ((size_t)n * H + h) * SS, dS, sizeof(double) * SS);
done:
    free(ckpt); free(prev); free(S); free(St); free(dS); free(dSt); free(p); free(u); free(du);
    free(dp); free(qn); free(kn); free(dqn); free(dkn);
    return rc;
}

static void *bwd_worker(void *arg)
{
    oracle_bwd_job *job = (oracle_bwd_job *)arg;
    const int64_t units = (int64_t)job->n_seqs * job->H;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        const int64_t i = job->next_unit++;
        pthread_mutex_unlock(&job->lock);
        if (i >= units) break;
        if (backward_unit(job, (int32_t)(i / job->H), (int32_t)(i % job->H)) != 0) {
            pthread_mutex_lock(&job->lock);
            job->failed = 1;
            pthread_mutex_unlock(&job->lock);
        }
    }
    return NULL;
}

/*
 * Gradients of L = sum d_out . out + sum d_final_state . final_state with respect to
 * every input of kda_oracle_forward_ex. d_final_state, initial_state and
 * d_initial_state may be NULL (zero / zero / not written). Gradient arrays have the
 * shapes of their inputs. Returns 0, or -1 on bad arguments or allocation failure.
 */
int kda_oracle_backward(const double *q, const double *k, const double *v,
                        const double *log_alpha, const double *beta, const int32_t *cu_seqlens,
                        const double *initial_state, int32_t qk_l2norm, const double *d_out,
                        const double *d_final_state, int32_t n_seqs, int32_t H, int32_t dk,
                        int32_t dv, double *dq, double *dkey, double *dval, double *dlog_alpha,
                        double *dbeta, double *d_initial_state, int32_t threads)
{
    if (!cu_seqlens || n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (cu_seqlens[0] != 0) return -1;
    for (int32_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !log_alpha || !beta || !d_out || !dq || !dkey ||
                                   !dval || !dlog_alpha || !dbeta))
        return -1;
    oracle_bwd_job job;
    memset(&job, 0, sizeof job);
    job.q = q; job.k = k; job.v = v; job.log_alpha = log_alpha; job.beta = beta;
    job.d_out = d_out; job.d_final_state = d_final_state; job.initial_state = initial_state;
    job.cu_seqlens = cu_seqlens; job.qk_l2norm = qk_l2norm; job.n_seqs = n_seqs; job.H = H;
    job.dk = dk; job.dv = dv; job.dq = dq; job.dkey = dkey; job.dval = dval;
    job.dlog_alpha = dlog_alpha; job.dbeta = dbeta; job.d_initial_state = d_initial_state;
    pthread_mutex_init(&job.lock, NULL);
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int i = 1; i < threads; ++i)
        if (pthread_create(&tid[started], NULL, bwd_worker, &job) == 0) ++started;
    bwd_worker(&job);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    pthread_mutex_destroy(&job.lock);
    return job.failed ? -1 : 0;
}
