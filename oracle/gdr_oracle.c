/*
 * gdr_oracle.c -- fp64, token-by-token reference for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY (see gdr_oracle.h).  Plain loops, no blocking, no
 * chunking, no log-space tricks: every function below follows the recurrence
 * as the pages state it so that it can be checked by eye.
 *
 * One step, for one (batch, head) slab with state S (dk x dv):
 *   a   = alpha_t                 (1 for DeltaNet, a broadcast scalar for Gated
 *                                  DeltaNet, a dk-vector for Kimi Delta Attention)
 *   S'  = Diag(a) S               decay first: Diag(alpha_t) multiplies S_{t-1}
 *                                 inside the product (KDA blog, section 2.1)
 *   e   = v_t - S'^T k_t          the write error: the written value minus what
 *                                 the memory already predicts for k_t (popular
 *                                 article on the study, the cross-layer section)
 *   u   = beta_t e
 *   S_t = S' + k_t u^T            which equals (I - beta k k^T) Diag(a) S + beta k v^T
 *   o_t = scale * S_t^T q_t       read-out after the write (KDA blog, section 2.1)
 */
#include "gdr_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* small helpers                                                              */
/* ------------------------------------------------------------------------- */

typedef struct {
    int64_t B, T, H, dk, dv;
    int gate;
    double scale;
    const double *q, *k, *v, *beta, *alpha, *S0, *dO, *dST;
    double *o, *ST, *dq, *dk_out, *dv_out, *dbeta, *dalpha, *dS0;
    double* E;        /* forward: write errors e_t, [B,T,H,dv] (NULL: not written) */
    const double* dE; /* backward: gradient arriving at e_t, [B,T,H,dv] (NULL: zero) */
    const double *erase, *write; /* Gated DeltaNet-2: erase and write gates, [B,T,H,dk] */
    int64_t N; /* decode: number of sequences */
    double* S; /* decode: state in/out */
    int status;
} job_t;

typedef struct {
    job_t* job;
    int tid, nthreads;
    void (*fn)(job_t*, int64_t slab);
} worker_t;

static void* worker_main(void* arg) {
    worker_t* w = (worker_t*)arg;
    int64_t nslab = (w->job->N > 0 ? w->job->N : w->job->B) * w->job->H;
    for (int64_t s = w->tid; s < nslab; s += w->nthreads) w->fn(w->job, s);
    return NULL;
}

/* Runs fn over every (b,h) slab on nthreads threads (static round robin). */
static int run_slabs(job_t* job, int nthreads, void (*fn)(job_t*, int64_t)) {
    int64_t nslab = (job->N > 0 ? job->N : job->B) * job->H;
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > nslab) nthreads = (int)(nslab > 0 ? nslab : 1);
    job->status = 0;
    if (nthreads == 1) {
        for (int64_t s = 0; s < nslab; ++s) fn(job, s);
        return job->status;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    worker_t* ws = (worker_t*)malloc(sizeof(worker_t) * (size_t)nthreads);
    if (!th || !ws) {
        free(th);
        free(ws);
        return -2;
    }
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        ws[i].job = job;
        ws[i].tid = i;
        ws[i].nthreads = nthreads;
        ws[i].fn = fn;
        if (pthread_create(&th[i], NULL, worker_main, &ws[i]) != 0) break;
        ++started;
    }
    /* threads that failed to start: run their share here */
    for (int i = started; i < nthreads; ++i) worker_main(&ws[i]);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    free(ws);
    return job->status;
}

/* The gate of token t for key channel i (1 for DeltaNet). */
static double gate_at(const job_t* j, int64_t b, int64_t t, int64_t h, int64_t i) {
    if (j->gate == ORACLE_GATE_NONE) return 1.0;
    if (j->gate == ORACLE_GATE_SCALAR) return j->alpha[(b * j->T + t) * j->H + h];
    return j->alpha[((b * j->T + t) * j->H + h) * j->dk + i];
}

/*
 * One recurrence step on a dk x dv state.
 *   S_prev: state before the token (read only); S_new: state after it.
 *   Also returns S' = Diag(a) S_prev (Sd), the write error e and u = beta e,
 *   which the adjoint needs.  a is the dk-vector of gates.
 */
static void step(int64_t dk, int64_t dv, const double* a, const double* kt, const double* vt,
                 double bt, const double* S_prev, double* Sd, double* e, double* u,
                 double* S_new) {
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) Sd[i * dv + j] = a[i] * S_prev[i * dv + j];
    for (int64_t j = 0; j < dv; ++j) {
        double p = 0.0; /* (S'^T k)_j */
        for (int64_t i = 0; i < dk; ++i) p += Sd[i * dv + j] * kt[i];
        e[j] = vt[j] - p;
        u[j] = bt * e[j];
    }
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) S_new[i * dv + j] = Sd[i * dv + j] + kt[i] * u[j];
}

static void readout(int64_t dk, int64_t dv, double scale, const double* S, const double* qt,
                    double* ot) {
    for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0; /* (S^T q)_j */
        for (int64_t i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i];
        ot[j] = scale * acc;
    }
}

/* ------------------------------------------------------------------------- */
/* forward                                                                    */
/* ------------------------------------------------------------------------- */

static void forward_slab(job_t* j, int64_t slab) {
    const int64_t b = slab / j->H, h = slab % j->H, dk = j->dk, dv = j->dv, T = j->T, H = j->H;
    const size_t nS = (size_t)(dk * dv);
    double* S = (double*)malloc(sizeof(double) * nS);
    double* Sn = (double*)malloc(sizeof(double) * nS);
    double* Sd = (double*)malloc(sizeof(double) * nS);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* e = (double*)malloc(sizeof(double) * (size_t)dv);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!S || !Sn || !Sd || !a || !e || !u) {
        j->status = -2;
        goto done;
    }
    if (j->S0)
        memcpy(S, j->S0 + (size_t)slab * nS, sizeof(double) * nS);
    else
        memset(S, 0, sizeof(double) * nS);
    for (int64_t t = 0; t < T; ++t) {
        const int64_t tok = (b * T + t) * H + h;
        for (int64_t i = 0; i < dk; ++i) a[i] = gate_at(j, b, t, h, i);
        step(dk, dv, a, j->k + tok * dk, j->v + tok * dv, j->beta[tok], S, Sd, e, u, Sn);
        if (j->E) memcpy(j->E + tok * dv, e, sizeof(double) * (size_t)dv);
        double* tmp = S;
        S = Sn;
        Sn = tmp;
        readout(dk, dv, j->scale, S, j->q + tok * dk, j->o + tok * dv);
    }
    if (j->ST) memcpy(j->ST + (size_t)slab * nS, S, sizeof(double) * nS);
done:
    free(S);
    free(Sn);
    free(Sd);
    free(a);
    free(e);
    free(u);
}

static int check_common(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate) {
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1) return -1;
    if (gate != ORACLE_GATE_NONE && gate != ORACLE_GATE_SCALAR && gate != ORACLE_GATE_CHANNEL)
        return -1;
    return 0;
}

int oracle_forward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate,
                   double scale, const double* q, const double* k, const double* v,
                   const double* beta, const double* alpha, const double* S0, double* o,
                   double* ST, int nthreads) {
    if (check_common(B, T, H, dk, dv, gate)) return -1;
    if (T > 0 && (!q || !k || !v || !beta || !o)) return -1;
    if (gate != ORACLE_GATE_NONE && T > 0 && !alpha) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.B = B; j.T = T; j.H = H; j.dk = dk; j.dv = dv; j.gate = gate; j.scale = scale;
    j.q = q; j.k = k; j.v = v; j.beta = beta; j.alpha = alpha; j.S0 = S0; j.o = o; j.ST = ST;
    return run_slabs(&j, nthreads, forward_slab);
}

int oracle_forward_errors(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate,
                          double scale, const double* q, const double* k, const double* v,
                          const double* beta, const double* alpha, const double* S0, double* o,
                          double* ST, double* E, int nthreads) {
    if (check_common(B, T, H, dk, dv, gate)) return -1;
    if (T > 0 && (!q || !k || !v || !beta || !o || !E)) return -1;
    if (gate != ORACLE_GATE_NONE && T > 0 && !alpha) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.B = B; j.T = T; j.H = H; j.dk = dk; j.dv = dv; j.gate = gate; j.scale = scale;
    j.q = q; j.k = k; j.v = v; j.beta = beta; j.alpha = alpha; j.S0 = S0; j.o = o; j.ST = ST;
    j.E = E;
    return run_slabs(&j, nthreads, forward_slab);
}

/* ------------------------------------------------------------------------- */
/* backward: adjoint of the token loop                                        */
/* ------------------------------------------------------------------------- */
/*
 * Reverse over t, carrying dS = dL/dS_t:
 *   dS    += scale q_t do_t^T           (o_t = scale S_t^T q_t)
 *   dq_t   = scale S_t do_t
 *   dk_t   = dS u,  du = dS^T k_t       (S_t = S' + k u^T)
 *   dbeta  = e . du, de = beta du       (u = beta e)
 *            (+ dE_t when the write error e_t itself is consumed downstream)
 *   dv_t   = de                         (e = v - S'^T k)
 *   dS'    = dS - k de^T,  dk_t -= S' de
 *   da_i   = sum_j dS'_ij S_{t-1,ij}    (S' = Diag(a) S_{t-1})
 *   dS     = Diag(a) dS'
 * States are recomputed from checkpoints taken every ceil(sqrt(T)) tokens.
 */
static void backward_slab(job_t* j, int64_t slab) {
    const int64_t b = slab / j->H, h = slab % j->H, dk = j->dk, dv = j->dv, T = j->T, H = j->H;
    const size_t nS = (size_t)(dk * dv);
    int64_t K = (int64_t)ceil(sqrt((double)(T > 0 ? T : 1)));
    if (K < 1) K = 1;
    const int64_t nseg = (T + K - 1) / K;
    double* ck = (double*)malloc(sizeof(double) * nS * (size_t)(nseg > 0 ? nseg : 1));
    double* buf = (double*)malloc(sizeof(double) * nS * (size_t)(K + 1));
    double* dS = (double*)malloc(sizeof(double) * nS);
    double* dSd = (double*)malloc(sizeof(double) * nS);
    double* Sd = (double*)malloc(sizeof(double) * nS);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* e = (double*)malloc(sizeof(double) * (size_t)dv);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    double* du = (double*)malloc(sizeof(double) * (size_t)dv);
    double* de = (double*)malloc(sizeof(double) * (size_t)dv);
    double* da = (double*)malloc(sizeof(double) * (size_t)dk);
    if (!ck || !buf || !dS || !dSd || !Sd || !a || !e || !u || !du || !de || !da) {
        j->status = -2;
        goto done;
    }
    /* forward pass: checkpoint the state before tokens 0, K, 2K, ... */
    {
        double* S = buf;
        double* Sn = buf + nS;
        if (j->S0)
            memcpy(S, j->S0 + (size_t)slab * nS, sizeof(double) * nS);
        else
            memset(S, 0, sizeof(double) * nS);
        for (int64_t t = 0; t < T; ++t) {
            if (t % K == 0) memcpy(ck + (size_t)(t / K) * nS, S, sizeof(double) * nS);
            const int64_t tok = (b * T + t) * H + h;
            for (int64_t i = 0; i < dk; ++i) a[i] = gate_at(j, b, t, h, i);
            step(dk, dv, a, j->k + tok * dk, j->v + tok * dv, j->beta[tok], S, Sd, e, u, Sn);
            double* tmp = S;
            S = Sn;
            Sn = tmp;
        }
    }
    if (j->dST)
        memcpy(dS, j->dST + (size_t)slab * nS, sizeof(double) * nS);
    else
        memset(dS, 0, sizeof(double) * nS);

    for (int64_t seg = nseg - 1; seg >= 0; --seg) {
        const int64_t t0 = seg * K, t1 = (t0 + K < T) ? t0 + K : T;
        /* buf[s] = state before token t0+s, buf[t1-t0] = state after token t1-1 */
        memcpy(buf, ck + (size_t)seg * nS, sizeof(double) * nS);
        for (int64_t t = t0; t < t1; ++t) {
            const int64_t tok = (b * T + t) * H + h;
            for (int64_t i = 0; i < dk; ++i) a[i] = gate_at(j, b, t, h, i);
            step(dk, dv, a, j->k + tok * dk, j->v + tok * dv, j->beta[tok],
                 buf + (size_t)(t - t0) * nS, Sd, e, u, buf + (size_t)(t - t0 + 1) * nS);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const int64_t tok = (b * T + t) * H + h;
            const double* qt = j->q + tok * dk;
            const double* kt = j->k + tok * dk;
            const double* vt = j->v + tok * dv;
            const double* dot = j->dO + tok * dv;
            const double bt = j->beta[tok];
            const double* Sprev = buf + (size_t)(t - t0) * nS;
            const double* Snew = buf + (size_t)(t - t0 + 1) * nS;
            double* dqt = j->dq + tok * dk;
            double* dkt = j->dk_out + tok * dk;
            double* dvt = j->dv_out + tok * dv;
            for (int64_t i = 0; i < dk; ++i) a[i] = gate_at(j, b, t, h, i);
            /* recompute S', e, u of this token */
            step(dk, dv, a, kt, vt, bt, Sprev, Sd, e, u, dSd /* scratch, overwritten below */);
            /* read-out */
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t jj = 0; jj < dv; ++jj) dS[i * dv + jj] += j->scale * qt[i] * dot[jj];
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t jj = 0; jj < dv; ++jj) acc += Snew[i * dv + jj] * dot[jj];
                dqt[i] = j->scale * acc;
            }
            /* write S_t = S' + k u^T */
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t jj = 0; jj < dv; ++jj) acc += dS[i * dv + jj] * u[jj];
                dkt[i] = acc;
            }
            double dbt = 0.0;
            for (int64_t jj = 0; jj < dv; ++jj) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i) acc += dS[i * dv + jj] * kt[i];
                du[jj] = acc;
                dbt += e[jj] * acc; /* u = beta e */
                de[jj] = bt * acc + (j->dE ? j->dE[tok * dv + jj] : 0.0);
                dvt[jj] = de[jj]; /* e = v - S'^T k */
            }
            j->dbeta[tok] = dbt;
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t jj = 0; jj < dv; ++jj) {
                    dSd[i * dv + jj] = dS[i * dv + jj] - kt[i] * de[jj];
                    acc += Sd[i * dv + jj] * de[jj];
                }
                dkt[i] -= acc;
            }
            /* decay S' = Diag(a) S_{t-1} */
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t jj = 0; jj < dv; ++jj) {
                    acc += dSd[i * dv + jj] * Sprev[i * dv + jj];
                    dS[i * dv + jj] = a[i] * dSd[i * dv + jj];
                }
                da[i] = acc;
            }
            if (j->gate == ORACLE_GATE_SCALAR) {
                double s = 0.0;
                for (int64_t i = 0; i < dk; ++i) s += da[i];
                if (j->dalpha) j->dalpha[tok] = s;
            } else if (j->gate == ORACLE_GATE_CHANNEL) {
                if (j->dalpha)
                    for (int64_t i = 0; i < dk; ++i) j->dalpha[tok * dk + i] = da[i];
            }
        }
    }
    if (j->dS0) memcpy(j->dS0 + (size_t)slab * nS, dS, sizeof(double) * nS);
done:
    free(ck);
    free(buf);
    free(dS);
    free(dSd);
    free(Sd);
    free(a);
    free(e);
    free(u);
    free(du);
    free(de);
    free(da);
}

int oracle_backward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate,
                    double scale, const double* q, const double* k, const double* v,
                    const double* beta, const double* alpha, const double* S0,
                    const double* dO, const double* dST, double* dq, double* dk_out,
                    double* dv_out, double* dbeta, double* dalpha, double* dS0, int nthreads) {
    if (check_common(B, T, H, dk, dv, gate)) return -1;
    if (T > 0 && (!q || !k || !v || !beta || !dO || !dq || !dk_out || !dv_out || !dbeta))
        return -1;
    if (gate != ORACLE_GATE_NONE && T > 0 && !alpha) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.B = B; j.T = T; j.H = H; j.dk = dk; j.dv = dv; j.gate = gate; j.scale = scale;
    j.q = q; j.k = k; j.v = v; j.beta = beta; j.alpha = alpha; j.S0 = S0;
    j.dO = dO; j.dST = dST; j.dq = dq; j.dk_out = dk_out; j.dv_out = dv_out;
    j.dbeta = dbeta; j.dalpha = dalpha; j.dS0 = dS0;
    return run_slabs(&j, nthreads, backward_slab);
}

int oracle_backward_errors(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate,
                           double scale, const double* q, const double* k, const double* v,
                           const double* beta, const double* alpha, const double* S0,
                           const double* dO, const double* dST, const double* dE, double* dq,
                           double* dk_out, double* dv_out, double* dbeta, double* dalpha,
                           double* dS0, int nthreads) {
    if (check_common(B, T, H, dk, dv, gate)) return -1;
    if (T > 0 && (!q || !k || !v || !beta || !dO || !dq || !dk_out || !dv_out || !dbeta))
        return -1;
    if (gate != ORACLE_GATE_NONE && T > 0 && !alpha) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.B = B; j.T = T; j.H = H; j.dk = dk; j.dv = dv; j.gate = gate; j.scale = scale;
    j.q = q; j.k = k; j.v = v; j.beta = beta; j.alpha = alpha; j.S0 = S0;
    j.dO = dO; j.dST = dST; j.dq = dq; j.dk_out = dk_out; j.dv_out = dv_out;
    j.dbeta = dbeta; j.dalpha = dalpha; j.dS0 = dS0; j.dE = dE;
    return run_slabs(&j, nthreads, backward_slab);
}

/* ------------------------------------------------------------------------- */
/* decode: one step per (sequence, head)                                      */
/* ------------------------------------------------------------------------- */

static void decode_slab(job_t* j, int64_t slab) {
    const int64_t dk = j->dk, dv = j->dv;
    const size_t nS = (size_t)(dk * dv);
    double* S = j->S + (size_t)slab * nS;
    double* Sd = (double*)malloc(sizeof(double) * nS);
    double* Sn = (double*)malloc(sizeof(double) * nS);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* e = (double*)malloc(sizeof(double) * (size_t)dv);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!Sd || !Sn || !a || !e || !u) {
        j->status = -2;
        goto done;
    }
    for (int64_t i = 0; i < dk; ++i) {
        if (j->gate == ORACLE_GATE_NONE)
            a[i] = 1.0;
        else if (j->gate == ORACLE_GATE_SCALAR)
            a[i] = j->alpha[slab];
        else
            a[i] = j->alpha[slab * dk + i];
    }
    step(dk, dv, a, j->k + slab * dk, j->v + slab * dv, j->beta[slab], S, Sd, e, u, Sn);
    memcpy(S, Sn, sizeof(double) * nS);
    readout(dk, dv, j->scale, S, j->q + slab * dk, j->o + slab * dv);
done:
    free(Sd);
    free(Sn);
    free(a);
    free(e);
    free(u);
}

int oracle_decode(int64_t N, int64_t H, int64_t dk, int64_t dv, int gate, double scale,
                  const double* q, const double* k, const double* v, const double* beta,
                  const double* alpha, double* S, double* o, int nthreads) {
    if (check_common(N, 1, H, dk, dv, gate)) return -1;
    if (N * H > 0 && (!q || !k || !v || !beta || !S || !o)) return -1;
    if (gate != ORACLE_GATE_NONE && N * H > 0 && !alpha) return -1;
    if (N == 0) return 0;
    job_t j;
    memset(&j, 0, sizeof j);
    j.N = N; j.H = H; j.T = 1; j.dk = dk; j.dv = dv; j.gate = gate; j.scale = scale;
    j.q = q; j.k = k; j.v = v; j.beta = beta; j.alpha = alpha; j.S = S; j.o = o;
    return run_slabs(&j, nthreads, decode_slab);
}

/* ------------------------------------------------------------------------- */
/* CLVR epilogue                                                              */
/* ------------------------------------------------------------------------- */

int oracle_clvr_forward(int64_t B, int64_t T, int64_t H, int64_t dv, const double* h_in,
                        const double* v, const double* lam, double* h_out) {
    if (B < 0 || T < 0 || H < 0 || dv < 1) return -1;
    if (B * T * H > 0 && (!h_in || !v || !h_out)) return -1;
    for (int64_t bt = 0; bt < B * T; ++bt)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t jj = 0; jj < dv; ++jj) {
                const int64_t c = h * dv + jj;
                const double l = lam ? lam[c] : 1.0;
                h_out[bt * H * dv + c] = h_in[bt * H * dv + c] + l * v[(bt * H + h) * dv + jj];
            }
    return 0;
}

int oracle_clvr_backward(int64_t B, int64_t T, int64_t H, int64_t dv, const double* dh,
                         const double* v, const double* lam, double* dv_acc, double* dlam) {
    if (B < 0 || T < 0 || H < 0 || dv < 1) return -1;
    if (B * T * H > 0 && (!dh || !v)) return -1;
    if (dlam)
        for (int64_t c = 0; c < H * dv; ++c) dlam[c] = 0.0;
    for (int64_t bt = 0; bt < B * T; ++bt)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t jj = 0; jj < dv; ++jj) {
                const int64_t c = h * dv + jj;
                const double g = dh[bt * H * dv + c];
                if (dv_acc) dv_acc[(bt * H + h) * dv + jj] += (lam ? lam[c] : 1.0) * g;
                if (dlam) dlam[c] += g * v[(bt * H + h) * dv + jj];
            }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Gated DeltaNet-2: separate erase and write gates                           */
/* ------------------------------------------------------------------------- */
/*
 * The popular article on the study (its Gated DeltaNet-2 paragraph) describes
 * this member only in words: erasing old content and writing new content are
 * decoupled and steered by two gates computed independently from the current
 * token, an erase gate choosing the regions of the memory to clear and a write
 * gate the regions to write; with the two gates equal the mechanism falls back
 * to Kimi Delta Attention, and further to Gated DeltaNet.  Reading taken (the
 * plainest one that keeps both reductions): the memory's regions are its key
 * channels (rows of S), the gates are dk-vectors e_t, w_t per token and head,
 * and one step is
 *   S'  = Diag(a) S                      decay first, as for the family
 *   p   = S'^T k_t                       what the memory predicts for k_t
 *   S_t = S' - (e_t * k_t) p^T + (w_t * k_t) v_t^T
 *       = (I - (e_t * k_t) k_t^T) Diag(a) S + (w_t * k_t) v_t^T
 *   o_t = scale * S_t^T q_t
 * (* elementwise).  e_t = w_t = beta_t 1 gives the step of oracle_forward.
 */
static void gdn2_step(int64_t dk, int64_t dv, const double* a, const double* kt, const double* vt,
                      const double* et, const double* wt, const double* S_prev, double* Sd, double* p,
                      double* S_new) {
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) Sd[i * dv + j] = a[i] * S_prev[i * dv + j];
    for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0; /* (S'^T k)_j */
        for (int64_t i = 0; i < dk; ++i) acc += Sd[i * dv + j] * kt[i];
        p[j] = acc;
    }
    for (int64_t i = 0; i < dk; ++i) {
        const double ek = et[i] * kt[i], wk = wt[i] * kt[i];
        for (int64_t j = 0; j < dv; ++j) S_new[i * dv + j] = Sd[i * dv + j] - ek * p[j] + wk * vt[j];
    }
}

static void gdn2_forward_slab(job_t* j, int64_t slab) {
    const int64_t b = slab / j->H, h = slab % j->H, dk = j->dk, dv = j->dv, T = j->T, H = j->H;
    const size_t nS = (size_t)(dk * dv);
    double* S = (double*)malloc(sizeof(double) * nS);
    double* Sn = (double*)malloc(sizeof(double) * nS);
    double* Sd = (double*)malloc(sizeof(double) * nS);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* p = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!S || !Sn || !Sd || !a || !p) {
        j->status = -2;
        goto done;
    }
    if (j->S0)
        memcpy(S, j->S0 + (size_t)slab * nS, sizeof(double) * nS);
    else
        memset(S, 0, sizeof(double) * nS);
    for (int64_t t = 0; t < T; ++t) {
        const int64_t tok = (b * T + t) * H + h;
        for (int64_t i = 0; i < dk; ++i) a[i] = gate_at(j, b, t, h, i);
        gdn2_step(dk, dv, a, j->k + tok * dk, j->v + tok * dv, j->erase + tok * dk, j->write + tok * dk, S, Sd,
                  p, Sn);
        double* tmp = S;
        S = Sn;
        Sn = tmp;
        readout(dk, dv, j->scale, S, j->q + tok * dk, j->o + tok * dv);
    }
    if (j->ST) memcpy(j->ST + (size_t)slab * nS, S, sizeof(double) * nS);
done:
    free(S);
    free(Sn);
    free(Sd);
    free(a);
    free(p);
}

int oracle_gdn2_forward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate, double scale,
                        const double* q, const double* k, const double* v, const double* erase,
                        const double* write, const double* alpha, const double* S0, double* o, double* ST,
                        int nthreads) {
    if (check_common(B, T, H, dk, dv, gate)) return -1;
    if (T > 0 && (!q || !k || !v || !erase || !write || !o)) return -1;
    if (gate != ORACLE_GATE_NONE && T > 0 && !alpha) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.B = B; j.T = T; j.H = H; j.dk = dk; j.dv = dv; j.gate = gate; j.scale = scale;
    j.q = q; j.k = k; j.v = v; j.erase = erase; j.write = write; j.alpha = alpha; j.S0 = S0; j.o = o;
    j.ST = ST;
    return run_slabs(&j, nthreads, gdn2_forward_slab);
}

static void gdn2_decode_slab(job_t* j, int64_t slab) {
    const int64_t n = slab / j->H, h = slab % j->H, dk = j->dk, dv = j->dv;
    const size_t nS = (size_t)(dk * dv);
    double* S = j->S + (size_t)slab * nS;
    double* Sn = (double*)malloc(sizeof(double) * nS);
    double* Sd = (double*)malloc(sizeof(double) * nS);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* p = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!Sn || !Sd || !a || !p) {
        j->status = -2;
        goto done;
    }
    for (int64_t i = 0; i < dk; ++i) a[i] = gate_at(j, n, 0, h, i);
    gdn2_step(dk, dv, a, j->k + slab * dk, j->v + slab * dv, j->erase + slab * dk, j->write + slab * dk, S, Sd,
              p, Sn);
    memcpy(S, Sn, sizeof(double) * nS);
    readout(dk, dv, j->scale, S, j->q + slab * dk, j->o + slab * dv);
done:
    free(Sn);
    free(Sd);
    free(a);
    free(p);
}

int oracle_gdn2_decode(int64_t N, int64_t H, int64_t dk, int64_t dv, int gate, double scale, const double* q,
                       const double* k, const double* v, const double* erase, const double* write,
                       const double* alpha, double* S, double* o, int nthreads) {
    if (check_common(N, 1, H, dk, dv, gate)) return -1;
    if (N * H > 0 && (!q || !k || !v || !erase || !write || !S || !o)) return -1;
    if (gate != ORACLE_GATE_NONE && N * H > 0 && !alpha) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.B = N; j.T = 1; j.H = H; j.dk = dk; j.dv = dv; j.gate = gate; j.scale = scale;
    j.q = q; j.k = k; j.v = v; j.erase = erase; j.write = write; j.alpha = alpha; j.S = S; j.o = o;
    j.N = N;
    return run_slabs(&j, nthreads, gdn2_decode_slab);
}
