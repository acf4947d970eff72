/*
 * kda_oracle.c -- fp64 token-by-token reference of the KDA operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links
 * or calls this file; only tests, the smoke check and the CPU-baseline leg of
 * the benchmark load it.  It shares no code with the HIP path.
 *
 * What it computes ("Kimi Linear" page, sections "Background: from the delta
 * rule to gated DeltaNet", "Kimi Delta Attention" and "The constrained DPLR
 * form and the chunkwise algorithm"):  the gated delta rule whose scalar
 * forget gate is replaced by a diagonal (per key channel) gate,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,            alpha_t = exp(log_alpha_t)  (elementwise),
 *
 * i.e. the DPLR transition Diag(alpha) - a b^T with a = beta k (the
 * learning-rate-scaled key) and b = alpha (.) k (the key modulated by the
 * gate).  Each step, literally in the order the page describes the delta rule:
 *   1. decay:      S <- Diag(alpha_t) S          (rows of S are key channels)
 *   2. read:       p = S^T k_t                   (what the memory predicts)
 *   3. correct:    u = beta_t (v_t - p)
 *   4. write:      S <- S + k_t u^T
 *   5. output:     o_t = S^T q_t                 (reads the updated state)
 *
 * Layout: tokens packed as [T_total, H, d] (row-major, d fastest); sequence s
 * is tokens cu_seqlens[s] .. cu_seqlens[s+1]-1.  State [N, H, dk, dv], dv
 * fastest.  q/k/v are fp32 or bf16 (uint16 bit patterns); bf16 values are
 * widened exactly, so the oracle sees the same real numbers the GPU reads.
 * A third input kind takes every per-token input (q, k, v, log_alpha, beta)
 * as fp64, for callers that form them in fp64 first.
 *
 * Threads: one (sequence, head) unit at a time per thread, pthreads.
 *
 * KDA_ORACLE_MUTANT (compile-time, tests only): plants one deliberate mistake
 * so the pin tests can show they catch it.  0 (default) is the correct oracle;
 * 1 decay after the write, 2 output before the write, 3 wrong sign of the
 * prediction, 4 transposed state in the output, 5 beta dropped, 6 gate used
 * without exp, 7 initial state ignored.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef KDA_ORACLE_MUTANT
#define KDA_ORACLE_MUTANT 0
#endif

typedef struct {
    int64_t num_seqs;
    const int64_t* cu;
    int heads, dk, dv;
    int in_bf16;
    const void *q, *k, *v;
    const void *log_alpha, *beta; /* fp32, or fp64 when in_bf16 == 2 */
    const double* init;
    double *out, *final_state;
    int64_t next_unit;
    pthread_mutex_t lock;
} job_t;

static double load_in(const void* p, int bf16, int64_t i) {
    if (bf16 == 2) return ((const double*)p)[i];
    if (bf16) {
        uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float*)p)[i];
}

static double load_gate(const job_t* J, int64_t i) {
    return J->in_bf16 == 2 ? ((const double*)J->log_alpha)[i] : (double)((const float*)J->log_alpha)[i];
}

static void run_unit(job_t* J, int64_t unit, double* S, double* kv, double* qv, double* vv,
                     double* av, double* u) {
    const int H = J->heads, dk = J->dk, dv = J->dv;
    const int64_t s = unit / H, h = unit % H;
    const int64_t t0 = J->cu[s], t1 = J->cu[s + 1];

    for (int64_t i = 0; i < (int64_t)dk * dv; ++i)
#if KDA_ORACLE_MUTANT == 7
        S[i] = 0.0; /* mutant: initial state ignored */
#else
        S[i] = J->init ? J->init[(s * H + h) * (int64_t)dk * dv + i] : 0.0;
#endif

    for (int64_t t = t0; t < t1; ++t) {
        const int64_t th = t * H + h;
        for (int c = 0; c < dk; ++c) {
            kv[c] = load_in(J->k, J->in_bf16, th * dk + c);
            qv[c] = load_in(J->q, J->in_bf16, th * dk + c);
#if KDA_ORACLE_MUTANT == 6
            av[c] = load_gate(J, th * dk + c); /* mutant: gate used without exp */
#else
            av[c] = exp(load_gate(J, th * dk + c));
#endif
        }
        for (int j = 0; j < dv; ++j) vv[j] = load_in(J->v, J->in_bf16, th * dv + j);
#if KDA_ORACLE_MUTANT == 5
        const double b = 1.0; /* mutant: beta dropped */
#else
        const double b = J->in_bf16 == 2 ? ((const double*)J->beta)[th] : (double)((const float*)J->beta)[th];
#endif

#if KDA_ORACLE_MUTANT != 1
        /* 1. decay the key-channel rows */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) S[c * dv + j] *= av[c];
#endif
        /* 2-3. read the prediction for k_t and form the correction */
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) u[j] += S[c * dv + j] * kv[c];
        for (int j = 0; j < dv; ++j) {
#if KDA_ORACLE_MUTANT == 3
            u[j] = b * (vv[j] + u[j]); /* mutant: wrong sign of the prediction */
#else
            u[j] = b * (vv[j] - u[j]);
#endif
        }
#if KDA_ORACLE_MUTANT == 2
        /* mutant: output taken from the state before the write */
        for (int j = 0; j < dv; ++j) {
            double o = 0.0;
            for (int c = 0; c < dk; ++c) o += S[c * dv + j] * qv[c];
            J->out[th * dv + j] = o;
        }
#endif
        /* 4. write the correction */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) S[c * dv + j] += kv[c] * u[j];
#if KDA_ORACLE_MUTANT == 1
        /* mutant: decay applied after the delta write instead of before */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) S[c * dv + j] *= av[c];
#endif
#if KDA_ORACLE_MUTANT != 2
        /* 5. output from the updated state */
        for (int j = 0; j < dv; ++j) {
            double o = 0.0;
#if KDA_ORACLE_MUTANT == 4
            /* mutant: transposed state (only meaningful for dk == dv) */
            for (int c = 0; c < dk; ++c) o += S[j * dv + c] * qv[c];
#else
            for (int c = 0; c < dk; ++c) o += S[c * dv + j] * qv[c];
#endif
            J->out[th * dv + j] = o;
        }
#endif
    }
    if (J->final_state) {
        double* F = J->final_state + (s * H + h) * (int64_t)dk * dv;
        memcpy(F, S, sizeof(double) * (size_t)dk * dv);
    }
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int dk = J->dk, dv = J->dv;
    const int dm = dk > dv ? dk : dv;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* buf = (double*)malloc(sizeof(double) * (size_t)5 * dm);
    if (!S || !buf) {
        free(S);
        free(buf);
        return (void*)1;
    }
    const int64_t units = J->num_seqs * J->heads;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t unit = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (unit >= units) break;
        run_unit(J, unit, S, buf, buf + dm, buf + 2 * dm, buf + 3 * dm, buf + 4 * dm);
    }
    free(S);
    free(buf);
    return NULL;
}

/*
 * kda_oracle_forward: run every (sequence, head) unit.
 *   cu_seqlens  int64 [num_seqs+1], non-decreasing, cu[0] = 0
 *   q, k        [T_total, heads, dk]  (fp32; bf16 bits if in_bf16 == 1; fp64 if 2)
 *   v           [T_total, heads, dv]
 *   log_alpha   [T_total, heads, dk];  beta [T_total, heads]  (fp32; fp64 if in_bf16 == 2)
 *   init_state  fp64 [num_seqs, heads, dk, dv] or NULL (zero)
 *   out         fp64 [T_total, heads, dv];  final_state fp64 [num_seqs, heads, dk, dv] or NULL
 * Returns 0 on success, nonzero on bad arguments or allocation failure.
 */
int kda_oracle_forward(int64_t num_seqs, const int64_t* cu_seqlens, int heads, int dk, int dv,
                       int in_bf16, const void* q, const void* k, const void* v,
                       const void* log_alpha, const void* beta, const double* init_state,
                       double* out, double* final_state, int nthreads) {
    if (num_seqs < 0 || heads <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return 1;
    if (cu_seqlens[0] != 0) return 1;
    for (int64_t s = 0; s < num_seqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return 1;
    if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !log_alpha || !beta || !out)) return 1;
    job_t J;
    J.num_seqs = num_seqs;
    J.cu = cu_seqlens;
    J.heads = heads;
    J.dk = dk;
    J.dv = dv;
    J.in_bf16 = in_bf16;
    J.q = q;
    J.k = k;
    J.v = v;
    J.log_alpha = log_alpha;
    J.beta = beta;
    J.init = init_state;
    J.out = out;
    J.final_state = final_state;
    J.next_unit = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int rc = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) {
        void* r = worker(&J);
        rc = r != NULL;
    }
    for (int i = 0; i < started; ++i) {
        void* r = NULL;
        pthread_join(th[i], &r);
        if (r) rc = 2;
    }
    pthread_mutex_destroy(&J.lock);
    return rc;
}

int kda_oracle_mutant(void) { return KDA_ORACLE_MUTANT; }

/*
 * Reverse mode of the same recurrence (the gradients of a loss L through every
 * token step above), fp64.  Per (sequence, head), with S_prev the state before
 * token t, S' = Diag(alpha) S_prev, p = S'^T k, u = beta (v - p),
 * S_t = S' + k u^T and o_t = S_t^T q, walking t backwards with dS = dL/dS_t:
 *     dS     += q do_t^T                       (o_t = S_t^T q)
 *     dq_t    = S_t do_t
 *     dk_t    = dS u ;  du = dS^T k            (S_t = S' + k u^T, dS' = dS)
 *     dbeta_t = du . (v - p) ;  dv_t = beta du ;  dp = -beta du
 *     dS'    += k dp^T ;  dk_t += S' dp        (p = S'^T k)
 *     dlog_alpha_t[c] = alpha_c sum_j S_prev[c][j] dS'[c][j]
 *     dS      = Diag(alpha) dS'                (dL/dS_prev)
 * and dL/dS_0 is dS after the first token.  States are checkpointed every 64
 * tokens on the way forward and each segment is recomputed before it is walked
 * back.  dO [T_total, heads, dv] and dS_final [num_seqs, heads, dk, dv] (or
 * NULL: zero) are fp64; inputs as for kda_oracle_forward; outputs fp64: dq, dk
 * [T_total, heads, dk], dv [T_total, heads, dv], dlog_alpha [T_total, heads,
 * dk], dbeta [T_total, heads], dS0 [num_seqs, heads, dk, dv].
 */
#define BWD_SEG 64

typedef struct {
    job_t f;
    const double *dO, *dS_final;
    double *dq, *dk, *dv, *dla, *dbeta, *dS0;
} bjob_t;

static void load_token(const job_t* J, int64_t th, double* kv, double* qv, double* vv, double* av, double* b) {
    const int dk = J->dk, dv = J->dv;
    for (int c = 0; c < dk; ++c) {
        kv[c] = load_in(J->k, J->in_bf16, th * dk + c);
        qv[c] = load_in(J->q, J->in_bf16, th * dk + c);
        av[c] = exp(load_gate(J, th * dk + c));
    }
    for (int j = 0; j < dv; ++j) vv[j] = load_in(J->v, J->in_bf16, th * dv + j);
    *b = J->in_bf16 == 2 ? ((const double*)J->beta)[th] : (double)((const float*)J->beta)[th];
}

/* one forward token step: S (state before) -> S (state after); u and p returned */
static void step_fwd(double* S, int dk, int dv, const double* kv, const double* vv, const double* av, double b,
                     double* p, double* u) {
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[c * dv + j] *= av[c];
    for (int j = 0; j < dv; ++j) p[j] = 0.0;
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) p[j] += S[c * dv + j] * kv[c];
    for (int j = 0; j < dv; ++j) u[j] = b * (vv[j] - p[j]);
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[c * dv + j] += kv[c] * u[j];
}

static int bwd_unit(bjob_t* B, int64_t unit) {
    job_t* J = &B->f;
    const int H = J->heads, dk = J->dk, dv = J->dv;
    const int64_t s = unit / H, h = unit % H;
    const int64_t t0 = J->cu[s], t1 = J->cu[s + 1], n = t1 - t0;
    const size_t SS = (size_t)dk * dv;
    const int64_t nseg = (n + BWD_SEG - 1) / BWD_SEG;
    double* ck = (double*)malloc(sizeof(double) * SS * (size_t)(nseg > 0 ? nseg : 1));  /* state before each segment */
    double* seg = (double*)malloc(sizeof(double) * SS * BWD_SEG);                      /* state before each token */
    double* S = (double*)malloc(sizeof(double) * SS);
    double* Sp = (double*)malloc(sizeof(double) * SS);  /* S' */
    double* dS = (double*)malloc(sizeof(double) * SS);
    const int dm = dk > dv ? dk : dv;
    double* buf = (double*)malloc(sizeof(double) * (size_t)dm * 8);
    if (!ck || !seg || !S || !Sp || !dS || !buf) {
        free(ck); free(seg); free(S); free(Sp); free(dS); free(buf);
        return 1;
    }
    double *kv = buf, *qv = buf + dm, *vv = buf + 2 * dm, *av = buf + 3 * dm, *p = buf + 4 * dm, *u = buf + 5 * dm,
           *du = buf + 6 * dm, *dp = buf + 7 * dm;
    double b;
    for (size_t i = 0; i < SS; ++i) S[i] = J->init ? J->init[(s * H + h) * SS + i] : 0.0;
    for (int64_t m = 0; m < nseg; ++m) {
        memcpy(ck + (size_t)m * SS, S, sizeof(double) * SS);
        const int64_t e = t0 + (m + 1) * BWD_SEG < t1 ? t0 + (m + 1) * BWD_SEG : t1;
        for (int64_t t = t0 + m * BWD_SEG; t < e; ++t) {
            load_token(J, t * H + h, kv, qv, vv, av, &b);
            step_fwd(S, dk, dv, kv, vv, av, b, p, u);
        }
    }
    for (size_t i = 0; i < SS; ++i) dS[i] = B->dS_final ? B->dS_final[(s * H + h) * SS + i] : 0.0;
    for (int64_t m = nseg - 1; m >= 0; --m) {
        const int64_t a = t0 + m * BWD_SEG, e = a + BWD_SEG < t1 ? a + BWD_SEG : t1;
        memcpy(S, ck + (size_t)m * SS, sizeof(double) * SS);
        for (int64_t t = a; t < e; ++t) {
            memcpy(seg + (size_t)(t - a) * SS, S, sizeof(double) * SS);
            load_token(J, t * H + h, kv, qv, vv, av, &b);
            step_fwd(S, dk, dv, kv, vv, av, b, p, u);
        }
        for (int64_t t = e - 1; t >= a; --t) {
            const int64_t th = t * H + h;
            const double* Sprev = seg + (size_t)(t - a) * SS;
            load_token(J, th, kv, qv, vv, av, &b);
            /* recompute S', p, u and S_t */
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j) Sp[c * dv + j] = av[c] * Sprev[c * dv + j];
            for (int j = 0; j < dv; ++j) p[j] = 0.0;
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j) p[j] += Sp[c * dv + j] * kv[c];
            for (int j = 0; j < dv; ++j) u[j] = b * (vv[j] - p[j]);
            const double* doo = B->dO + th * dv;
            /* output: dS += q do^T, dq = S_t do with S_t = S' + k u^T */
            for (int c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) {
                    acc += (Sp[c * dv + j] + kv[c] * u[j]) * doo[j];
                    dS[c * dv + j] += qv[c] * doo[j];
                }
                B->dq[th * dk + c] = acc;
            }
            /* write: dk = dS u, du = dS^T k */
            for (int j = 0; j < dv; ++j) du[j] = 0.0;
            for (int c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) {
                    acc += dS[c * dv + j] * u[j];
                    du[j] += dS[c * dv + j] * kv[c];
                }
                B->dk[th * dk + c] = acc;
            }
            /* correction: dbeta, dv, dp */
            double db = 0.0;
            for (int j = 0; j < dv; ++j) {
                db += du[j] * (vv[j] - p[j]);
                B->dv[th * dv + j] = b * du[j];
                dp[j] = -b * du[j];
            }
            B->dbeta[th] = db;
            /* prediction: dS' = dS + k dp^T, dk += S' dp */
            for (int c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) {
                    dS[c * dv + j] += kv[c] * dp[j];
                    acc += Sp[c * dv + j] * dp[j];
                }
                B->dk[th * dk + c] += acc;
            }
            /* decay: dlog_alpha, dS_prev = Diag(alpha) dS' */
            for (int c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += Sprev[c * dv + j] * dS[c * dv + j];
                B->dla[th * dk + c] = av[c] * acc;
                for (int j = 0; j < dv; ++j) dS[c * dv + j] *= av[c];
            }
        }
    }
    memcpy(B->dS0 + (s * H + h) * SS, dS, sizeof(double) * SS);
    free(ck); free(seg); free(S); free(Sp); free(dS); free(buf);
    return 0;
}

static void* bwd_worker(void* arg) {
    bjob_t* B = (bjob_t*)arg;
    job_t* J = &B->f;
    const int64_t units = J->num_seqs * J->heads;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t unit = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (unit >= units) break;
        if (bwd_unit(B, unit)) return (void*)1;
    }
    return NULL;
}

int kda_oracle_backward(int64_t num_seqs, const int64_t* cu_seqlens, int heads, int dk, int dv, int in_bf16,
                        const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                        const double* init_state, const double* dO, const double* dS_final, double* dq,
                        double* dk_out, double* dv_out, double* dla, double* dbeta, double* dS0, int nthreads) {
    if (num_seqs < 0 || heads <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens || cu_seqlens[0] != 0) return 1;
    for (int64_t s = 0; s < num_seqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return 1;
    if (!dS0) return 1;
    if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !log_alpha || !beta || !dO || !dq || !dk_out || !dv_out ||
                                     !dla || !dbeta))
        return 1;
    bjob_t B;
    memset(&B, 0, sizeof B);
    B.f.num_seqs = num_seqs;
    B.f.cu = cu_seqlens;
    B.f.heads = heads;
    B.f.dk = dk;
    B.f.dv = dv;
    B.f.in_bf16 = in_bf16;
    B.f.q = q;
    B.f.k = k;
    B.f.v = v;
    B.f.log_alpha = log_alpha;
    B.f.beta = beta;
    B.f.init = init_state;
    B.f.next_unit = 0;
    B.dO = dO;
    B.dS_final = dS_final;
    B.dq = dq;
    B.dk = dk_out;
    B.dv = dv_out;
    B.dla = dla;
    B.dbeta = dbeta;
    B.dS0 = dS0;
    pthread_mutex_init(&B.f.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int rc = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, bwd_worker, &B) != 0) break;
        ++started;
    }
    if (started == 0) rc = bwd_worker(&B) != NULL;
    for (int i = 0; i < started; ++i) {
        void* r = NULL;
        pthread_join(th[i], &r);
        if (r) rc = 2;
    }
    pthread_mutex_destroy(&B.f.lock);
    return rc;
}

/* ------------------------------------------------------------------------
 * General DPLR transition (the baseline KDA constrains; "Kimi Linear" page,
 * section "The constrained DPLR form and the chunkwise algorithm"): a
 * diagonal gate plus a rank-one term with two independent vectors a_t, b_t,
 *
 *     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,    o_t = S_t^T q_t.
 *
 * KDA is the case a = beta k, b = alpha (.) k with write key beta k.  Each
 * step, in this order:
 *   1. read:    p = S^T b_t          (from the state the step starts from)
 *   2. decay:   S <- Diag(alpha_t) S
 *   3. correct: S <- S - a_t p^T
 *   4. write:   S <- S + k_t v_t^T
 *   5. output:  o_t = S^T q_t
 * Inputs as for kda_oracle_forward, with a and b laid out like k and no beta.
 *
 * KDA_ORACLE_MUTANT 8: b reads the decayed state (steps 1 and 2 swapped);
 * 9: the roles of a and b exchanged (S <- S - b (a^T S)).
 * ------------------------------------------------------------------------ */
typedef struct {
    int64_t num_seqs;
    const int64_t* cu;
    int heads, dk, dv;
    int in_bf16;
    const void *q, *k, *v, *a, *b;
    const float* log_alpha;
    const double* init;
    double *out, *final_state;
    int64_t next_unit;
    pthread_mutex_t lock;
} djob_t;

static void dplr_unit(djob_t* J, int64_t unit, double* S, double* buf) {
    const int H = J->heads, dk = J->dk, dv = J->dv;
    const int64_t s = unit / H, h = unit % H;
    const int64_t t0 = J->cu[s], t1 = J->cu[s + 1];
    double *qv = buf, *kv = buf + dk, *av = buf + 2 * dk, *bv = buf + 3 * dk, *al = buf + 4 * dk;
    double *vv = buf + 5 * dk, *p = vv + dv;
    for (int64_t i = 0; i < (int64_t)dk * dv; ++i)
        S[i] = J->init ? J->init[(s * H + h) * (int64_t)dk * dv + i] : 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t th = t * H + h;
        for (int c = 0; c < dk; ++c) {
            qv[c] = load_in(J->q, J->in_bf16, th * dk + c);
            kv[c] = load_in(J->k, J->in_bf16, th * dk + c);
            av[c] = load_in(J->a, J->in_bf16, th * dk + c);
            bv[c] = load_in(J->b, J->in_bf16, th * dk + c);
            al[c] = exp((double)J->log_alpha[th * dk + c]);
        }
        for (int j = 0; j < dv; ++j) vv[j] = load_in(J->v, J->in_bf16, th * dv + j);
#if KDA_ORACLE_MUTANT == 8
        for (int c = 0; c < dk; ++c) /* mutant: decay before the read */
            for (int j = 0; j < dv; ++j) S[c * dv + j] *= al[c];
#endif
        /* 1. read through b */
        const double* rd = bv;
#if KDA_ORACLE_MUTANT == 9
        rd = av; /* mutant: a and b exchanged */
#endif
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) p[j] += rd[c] * S[c * dv + j];
#if KDA_ORACLE_MUTANT != 8
        /* 2. decay */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) S[c * dv + j] *= al[c];
#endif
        /* 3-4. rank-one correction along a, then the write */
        const double* wr = av;
#if KDA_ORACLE_MUTANT == 9
        wr = bv;
#endif
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) S[c * dv + j] += kv[c] * vv[j] - wr[c] * p[j];
        /* 5. output */
        for (int j = 0; j < dv; ++j) {
            double o = 0.0;
            for (int c = 0; c < dk; ++c) o += S[c * dv + j] * qv[c];
            J->out[th * dv + j] = o;
        }
    }
    if (J->final_state) memcpy(J->final_state + (s * H + h) * (int64_t)dk * dv, S, sizeof(double) * (size_t)dk * dv);
}

static void* dplr_worker(void* arg) {
    djob_t* J = (djob_t*)arg;
    double* S = (double*)malloc(sizeof(double) * (size_t)J->dk * J->dv);
    double* buf = (double*)malloc(sizeof(double) * ((size_t)5 * J->dk + 2 * (size_t)J->dv));
    if (!S || !buf) {
        free(S);
        free(buf);
        return (void*)1;
    }
    const int64_t units = J->num_seqs * J->heads;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t unit = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (unit >= units) break;
        dplr_unit(J, unit, S, buf);
    }
    free(S);
    free(buf);
    return NULL;
}

/*
 * dplr_oracle_forward: every (sequence, head) unit of the general DPLR recurrence.
 *   q, k, a, b  [T_total, heads, dk];  v [T_total, heads, dv]  (fp32, or bf16 bits if in_bf16)
 *   log_alpha   fp32 [T_total, heads, dk]
 *   init_state, out, final_state as for kda_oracle_forward.
 */
int dplr_oracle_forward(int64_t num_seqs, const int64_t* cu_seqlens, int heads, int dk, int dv, int in_bf16,
                        const void* q, const void* k, const void* v, const void* a, const void* b,
                        const float* log_alpha, const double* init_state, double* out, double* final_state,
                        int nthreads) {
    if (num_seqs < 0 || heads <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens || (in_bf16 != 0 && in_bf16 != 1)) return 1;
    if (cu_seqlens[0] != 0) return 1;
    for (int64_t s = 0; s < num_seqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return 1;
    if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !a || !b || !log_alpha || !out)) return 1;
    djob_t J;
    J.num_seqs = num_seqs;
    J.cu = cu_seqlens;
    J.heads = heads;
    J.dk = dk;
    J.dv = dv;
    J.in_bf16 = in_bf16;
    J.q = q;
    J.k = k;
    J.v = v;
    J.a = a;
    J.b = b;
    J.log_alpha = log_alpha;
    J.init = init_state;
    J.out = out;
    J.final_state = final_state;
    J.next_unit = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int rc = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, dplr_worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) {
        if (dplr_worker(&J) != NULL) rc = 2;
    }
    for (int i = 0; i < started; ++i) {
        void* r = NULL;
        pthread_join(th[i], &r);
        if (r != NULL) rc = 2;
    }
    pthread_mutex_destroy(&J.lock);
    return rc;
}
