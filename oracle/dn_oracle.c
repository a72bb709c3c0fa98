/*
 * dn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential fp64 evaluation of the gated delta rule and of its
 * hand-derived reverse-mode pass.  It is the correctness oracle for the HIP
 * library: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no code with the GPU path.
 *
 * What it computes (per independent head; state S is d_v x d_k, read out as
 * o_t = S_t q_t):
 *
 *   a_t   = exp(g_t)                 per-channel decay, g_t the log-decay:
 *                                     gate 0: none (a_t = 1, DeltaNet),
 *                                     gate 1: one scalar per step (Gated DeltaNet),
 *                                     gate 2: one value per key channel (KDA)
 *   Sbar  = S_{t-1} Diag(a_t)          decay first ...
 *   p_t   = Sbar k_t                   ... then the delta (online-regression) step
 *   u_t   = beta_t (v_t - p_t)
 *   S_t   = Sbar + u_t k_t^T           = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   o_t   = S_t q_t                    read-after-write
 *
 * Sources: ReWY abstract (delta-rule linear attention for DeltaNet, GDN, KDA;
 * chunkwise forms preserve the recurrence and its gradients exactly); the SFDA
 * technical summary, "Kernarchitektur" (recurrence S_t = (I - beta k k*) Lambda_t
 * S_{t-1} + beta k v*, Lambda_t = diag(alpha_t ...): this is its transpose, with
 * zero phase, i.e. KDA); the KLA abstract (GDN = gated decay + delta-rule residual
 * write, an online-regression objective); the Fast Weight Attention abstract
 * (read-after-write semantics).
 *
 * Reverse mode: for cotangents dO (and dhT on the final state) it returns the
 * vector-Jacobian products dq, dk, dv, dbeta, dg, dh0 of
 *   L = <O, dO> + <hT, dhT>.
 * It walks the steps backwards; states are checkpointed every SEG steps in the
 * forward sweep and each segment is recomputed from its checkpoint.
 *
 * Layouts (row-major, heads independent, BH = batch*heads):
 *   q, k, dq, dk : [BH][T][dk]      v, o, dO, dv : [BH][T][dv]
 *   beta, dbeta  : [BH][T]          g, dg : [BH][T] (gate 1) or [BH][T][dk] (gate 2)
 *   h0, hT, dh0, dhT : [BH][dv][dk]
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define SEG 64

typedef struct {
    int T, dk, dv, gate;
    const double *q, *k, *v, *beta, *g, *h0, *dout, *dhT;
    double *o, *hT;
    double *dq, *dkk, *dvv, *dbeta, *dg, *dh0;
} head_t;

/* decay vector a (length dk) of step t */
static void decay_of_step(const head_t *h, int t, double *a)
{
    int c;
    for (c = 0; c < h->dk; ++c) {
        if (h->gate == 0)
            a[c] = 1.0;
        else if (h->gate == 1)
            a[c] = exp(h->g[t]);
        else
            a[c] = exp(h->g[(size_t)t * h->dk + c]);
    }
}

/*
 * One forward step: Sprev -> S (the two may not alias).  Also leaves the
 * decay a, the decayed state Sbar, the prediction p and the write u of the step
 * in the scratch arrays (the reverse pass reads them).
 */
static void step_forward(const head_t *h, int t, const double *Sprev, double *S,
                         double *a, double *Sbar, double *p, double *u)
{
    const int dk = h->dk, dv = h->dv;
    const double *kt = h->k + (size_t)t * dk;
    const double *vt = h->v + (size_t)t * dv;
    const double bt = h->beta[t];
    int i, c;
    decay_of_step(h, t, a);
    for (i = 0; i < dv; ++i) {
        const double *srow = Sprev + (size_t)i * dk;
        double *brow = Sbar + (size_t)i * dk;
        double acc = 0.0;
        for (c = 0; c < dk; ++c) {
            brow[c] = srow[c] * a[c];
            acc += brow[c] * kt[c];
        }
        p[i] = acc;
        u[i] = bt * (vt[i] - acc);
    }
    for (i = 0; i < dv; ++i) {
        const double *brow = Sbar + (size_t)i * dk;
        double *row = S + (size_t)i * dk;
        for (c = 0; c < dk; ++c)
            row[c] = brow[c] + u[i] * kt[c];
    }
}

static void read_out(const head_t *h, int t, const double *S, double *ot)
{
    const int dk = h->dk, dv = h->dv;
    const double *qt = h->q + (size_t)t * dk;
    int i, c;
    for (i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (c = 0; c < dk; ++c)
            acc += S[(size_t)i * dk + c] * qt[c];
        ot[i] = acc;
    }
}

static int head_forward(head_t *h)
{
    const int dk = h->dk, dv = h->dv;
    const size_t ns = (size_t)dk * dv;
    double *S = calloc(ns, sizeof(double)), *Sn = calloc(ns, sizeof(double));
    double *Sbar = calloc(ns, sizeof(double));
    double *a = calloc((size_t)dk, sizeof(double));
    double *p = calloc((size_t)dv, sizeof(double)), *u = calloc((size_t)dv, sizeof(double));
    int t;
    if (!S || !Sn || !Sbar || !a || !p || !u) {
        free(S); free(Sn); free(Sbar); free(a); free(p); free(u);
        return -1;
    }
    if (h->h0)
        memcpy(S, h->h0, ns * sizeof(double));
    for (t = 0; t < h->T; ++t) {
        double *tmp;
        step_forward(h, t, S, Sn, a, Sbar, p, u);
        tmp = S; S = Sn; Sn = tmp;
        if (h->o)
            read_out(h, t, S, h->o + (size_t)t * dv);
    }
    if (h->hT)
        memcpy(h->hT, S, ns * sizeof(double));
    free(S); free(Sn); free(Sbar); free(a); free(p); free(u);
    return 0;
}

/*
 * Reverse mode.  Each step t, walked from T-1 down to 0, given dS = dL/dS_t:
 *   dS    += do_t q_t^T              dq_t  = S_t^T do_t                (o_t = S_t q_t)
 *   du     = dS k_t                  dk_t  = dS^T u_t                  (S_t = Sbar + u k^T)
 *   dbeta_t= du . (v_t - p_t)        dv_t  = beta_t du   dp = -beta_t du   (u = beta (v - p))
 *   dSbar  = dS + dp k_t^T           dk_t += Sbar^T dp                 (p = Sbar k)
 *   dg_t[c]= sum_i Sbar[i,c] dSbar[i,c]   (gate 1: summed over c too)  (Sbar = S_{t-1} Diag(e^g))
 *   dS_{t-1} = dSbar Diag(a_t)
 */
static int head_backward(head_t *h)
{
    const int T = h->T, dk = h->dk, dv = h->dv;
    const size_t ns = (size_t)dk * dv;
    const int nseg = (T + SEG - 1) / SEG;
    double *ckpt = malloc(((size_t)(nseg > 0 ? nseg : 1)) * ns * sizeof(double));
    double *Sseg = malloc((size_t)(SEG + 1) * ns * sizeof(double));
    double *S = calloc(ns, sizeof(double)), *Sn = calloc(ns, sizeof(double));
    double *Sbar = calloc(ns, sizeof(double)), *dS = calloc(ns, sizeof(double));
    double *a = calloc((size_t)dk, sizeof(double));
    double *p = calloc((size_t)dv, sizeof(double)), *u = calloc((size_t)dv, sizeof(double));
    double *du = calloc((size_t)dv, sizeof(double)), *dp = calloc((size_t)dv, sizeof(double));
    int t, s, i, c;
    int rc = 0;
    if (!ckpt || !Sseg || !S || !Sn || !Sbar || !dS || !a || !p || !u || !du || !dp) {
        rc = -1;
        goto out;
    }
    /* forward sweep, checkpointing the state that enters each segment */
    if (h->h0)
        memcpy(S, h->h0, ns * sizeof(double));
    for (t = 0; t < T; ++t) {
        double *tmp;
        if (t % SEG == 0)
            memcpy(ckpt + (size_t)(t / SEG) * ns, S, ns * sizeof(double));
        step_forward(h, t, S, Sn, a, Sbar, p, u);
        tmp = S; S = Sn; Sn = tmp;
    }
    if (h->dhT)
        memcpy(dS, h->dhT, ns * sizeof(double));
    for (s = nseg - 1; s >= 0; --s) {
        const int t0 = s * SEG;
        const int t1 = (t0 + SEG < T) ? t0 + SEG : T;
        /* recompute the segment: Sseg[j] = state before step t0 + j */
        memcpy(Sseg, ckpt + (size_t)s * ns, ns * sizeof(double));
        for (t = t0; t < t1; ++t)
            step_forward(h, t, Sseg + (size_t)(t - t0) * ns, Sseg + (size_t)(t - t0 + 1) * ns,
                         a, Sbar, p, u);
        for (t = t1 - 1; t >= t0; --t) {
            const double *Sprev = Sseg + (size_t)(t - t0) * ns;
            const double *St = Sseg + (size_t)(t - t0 + 1) * ns;
            const double *qt = h->q + (size_t)t * dk;
            const double *kt = h->k + (size_t)t * dk;
            const double *vt = h->v + (size_t)t * dv;
            const double *dot = h->dout ? h->dout + (size_t)t * dv : NULL;
            double *dqt = h->dq + (size_t)t * dk;
            double *dkt = h->dkk + (size_t)t * dk;
            double *dvt = h->dvv + (size_t)t * dv;
            const double bt = h->beta[t];
            double db = 0.0;
            step_forward(h, t, Sprev, Sn, a, Sbar, p, u); /* Sbar, p, u of step t */
            /* o_t = S_t q_t */
            for (c = 0; c < dk; ++c)
                dqt[c] = 0.0;
            if (dot) {
                for (i = 0; i < dv; ++i)
                    for (c = 0; c < dk; ++c) {
                        dS[(size_t)i * dk + c] += dot[i] * qt[c];
                        dqt[c] += St[(size_t)i * dk + c] * dot[i];
                    }
            }
            /* S_t = Sbar + u k^T */
            for (i = 0; i < dv; ++i) {
                double acc = 0.0;
                for (c = 0; c < dk; ++c)
                    acc += dS[(size_t)i * dk + c] * kt[c];
                du[i] = acc;
            }
            for (c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (i = 0; i < dv; ++i)
                    acc += dS[(size_t)i * dk + c] * u[i];
                dkt[c] = acc;
            }
            /* u = beta (v - p) */
            for (i = 0; i < dv; ++i) {
                db += du[i] * (vt[i] - p[i]);
                dvt[i] = bt * du[i];
                dp[i] = -bt * du[i];
            }
            h->dbeta[t] = db;
            /* p = Sbar k: dSbar = dS + dp k^T, dk += Sbar^T dp */
            for (i = 0; i < dv; ++i)
                for (c = 0; c < dk; ++c)
                    dS[(size_t)i * dk + c] += dp[i] * kt[c];
            for (c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (i = 0; i < dv; ++i)
                    acc += Sbar[(size_t)i * dk + c] * dp[i];
                dkt[c] += acc;
            }
            /* Sbar = S_{t-1} Diag(a): dS now holds dSbar */
            if (h->gate == 1) {
                double acc = 0.0;
                for (i = 0; i < dv; ++i)
                    for (c = 0; c < dk; ++c)
                        acc += Sbar[(size_t)i * dk + c] * dS[(size_t)i * dk + c];
                h->dg[t] = acc;
            } else if (h->gate == 2) {
                for (c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (i = 0; i < dv; ++i)
                        acc += Sbar[(size_t)i * dk + c] * dS[(size_t)i * dk + c];
                    h->dg[(size_t)t * dk + c] = acc;
                }
            }
            for (i = 0; i < dv; ++i)
                for (c = 0; c < dk; ++c)
                    dS[(size_t)i * dk + c] *= a[c];
        }
    }
    if (h->dh0)
        memcpy(h->dh0, dS, ns * sizeof(double));
out:
    free(ckpt); free(Sseg); free(S); free(Sn); free(Sbar); free(dS);
    free(a); free(p); free(u); free(du); free(dp);
    return rc;
}

/* ---- thread pool over heads ------------------------------------------------ */

typedef struct {
    head_t *heads;
    int nheads;
    int backward;
    int next;
    int failed;
    pthread_mutex_t mu;
} pool_t;

static void *worker(void *arg)
{
    pool_t *pl = (pool_t *)arg;
    for (;;) {
        int idx, rc;
        pthread_mutex_lock(&pl->mu);
        idx = pl->next++;
        pthread_mutex_unlock(&pl->mu);
        if (idx >= pl->nheads)
            break;
        rc = pl->backward ? head_backward(&pl->heads[idx]) : head_forward(&pl->heads[idx]);
        if (rc) {
            pthread_mutex_lock(&pl->mu);
            pl->failed = 1;
            pthread_mutex_unlock(&pl->mu);
        }
    }
    return NULL;
}

static int run_pool(head_t *heads, int nheads, int backward, int nthreads)
{
    pool_t pl;
    pthread_t *th;
    int i, nt;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    nt = nthreads < nheads ? nthreads : nheads;
    if (nt < 1)
        nt = 1;
    pl.heads = heads;
    pl.nheads = nheads;
    pl.backward = backward;
    pl.next = 0;
    pl.failed = 0;
    pthread_mutex_init(&pl.mu, NULL);
    th = malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th)
        return -1;
    for (i = 0; i < nt; ++i)
        if (pthread_create(&th[i], NULL, worker, &pl)) {
            nt = i;
            pl.failed = 1;
            break;
        }
    for (i = 0; i < nt; ++i)
        pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&pl.mu);
    return pl.failed ? -1 : 0;
}

static void fill_head(head_t *h, int b, int T, int dk, int dv, int gate,
                      const double *q, const double *k, const double *v, const double *beta,
                      const double *g, const double *h0)
{
    const size_t tk = (size_t)T * dk, tv = (size_t)T * dv, ns = (size_t)dk * dv;
    memset(h, 0, sizeof(*h));
    h->T = T; h->dk = dk; h->dv = dv; h->gate = gate;
    h->q = q + b * tk;
    h->k = k + b * tk;
    h->v = v + b * tv;
    h->beta = beta + (size_t)b * T;
    h->g = gate == 0 ? NULL : (gate == 1 ? g + (size_t)b * T : g + b * tk);
    h->h0 = h0 ? h0 + b * ns : NULL;
}

/* Returns 0 on success, -1 on bad arguments or allocation failure. */
int dn_oracle_fwd(int BH, int T, int dk, int dv, int gate,
                  const double *q, const double *k, const double *v, const double *beta,
                  const double *g, const double *h0, double *o, double *hT, int nthreads)
{
    head_t *heads;
    int b, rc;
    if (BH < 0 || T < 0 || dk <= 0 || dv <= 0 || gate < 0 || gate > 2)
        return -1;
    if (gate != 0 && !g)
        return -1;
    if (BH == 0)
        return 0;
    heads = calloc((size_t)BH, sizeof(head_t));
    if (!heads)
        return -1;
    for (b = 0; b < BH; ++b) {
        fill_head(&heads[b], b, T, dk, dv, gate, q, k, v, beta, g, h0);
        heads[b].o = o ? o + (size_t)b * T * dv : NULL;
        heads[b].hT = hT ? hT + (size_t)b * dk * dv : NULL;
    }
    rc = run_pool(heads, BH, 0, nthreads);
    free(heads);
    return rc;
}

int dn_oracle_bwd(int BH, int T, int dk, int dv, int gate,
                  const double *q, const double *k, const double *v, const double *beta,
                  const double *g, const double *h0, const double *dout, const double *dhT,
                  double *dq, double *dkk, double *dvv, double *dbeta, double *dg, double *dh0,
                  int nthreads)
{
    head_t *heads;
    int b, rc;
    if (BH < 0 || T < 0 || dk <= 0 || dv <= 0 || gate < 0 || gate > 2)
        return -1;
    if (gate != 0 && (!g || !dg))
        return -1;
    if (!dq || !dkk || !dvv || !dbeta)
        return -1;
    if (BH == 0)
        return 0;
    heads = calloc((size_t)BH, sizeof(head_t));
    if (!heads)
        return -1;
    for (b = 0; b < BH; ++b) {
        const size_t tk = (size_t)T * dk, tv = (size_t)T * dv, ns = (size_t)dk * dv;
        fill_head(&heads[b], b, T, dk, dv, gate, q, k, v, beta, g, h0);
        heads[b].dout = dout ? dout + b * tv : NULL;
        heads[b].dhT = dhT ? dhT + b * ns : NULL;
        heads[b].dq = dq + b * tk;
        heads[b].dkk = dkk + b * tk;
        heads[b].dvv = dvv + b * tv;
        heads[b].dbeta = dbeta + (size_t)b * T;
        heads[b].dg = gate == 0 ? NULL : (gate == 1 ? dg + (size_t)b * T : dg + b * tk);
        heads[b].dh0 = dh0 ? dh0 + b * ns : NULL;
    }
    rc = run_pool(heads, BH, 1, nthreads);
    free(heads);
    return rc;
}
