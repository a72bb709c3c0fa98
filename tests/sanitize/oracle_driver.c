/* Runs the C oracle's forward and reverse mode on small problems of every gate,
 * with odd sizes (sequences that end inside a checkpoint segment, d_k != d_v),
 * optional arguments left NULL, one and several threads, and its argument
 * checks -- built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py, which fails on any report. */
#include <stdio.h>
#include <stdlib.h>

int dn_oracle_fwd(int BH, int T, int dk, int dv, int gate, const double *q, const double *k, const double *v,
                  const double *beta, const double *g, const double *h0, double *o, double *hT, int nthreads);
int dn_oracle_bwd(int BH, int T, int dk, int dv, int gate, const double *q, const double *k, const double *v,
                  const double *beta, const double *g, const double *h0, const double *dout, const double *dhT,
                  double *dq, double *dkk, double *dvv, double *dbeta, double *dg, double *dh0, int nthreads);

static double *arr(size_t n, unsigned *seed, double scale)
{
    double *x = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) {
        *seed = *seed * 1103515245u + 12345u;
        x[i] = scale * (((*seed >> 8) & 0xffff) / 32768.0 - 1.0);
    }
    return x;
}

static int run(int BH, int T, int dk, int dv, int gate, int with_h0, int with_dhT, int nthreads)
{
    unsigned s = 1234u + (unsigned)(BH * 7 + T * 3 + dk + gate);
    const size_t tk = (size_t)BH * T * dk, tv = (size_t)BH * T * dv, ns = (size_t)BH * dk * dv;
    const size_t ng = gate == 0 ? 0 : (gate == 1 ? (size_t)BH * T : tk);
    double *q = arr(tk, &s, 0.3), *k = arr(tk, &s, 0.3), *v = arr(tv, &s, 1.0), *beta = arr((size_t)BH * T, &s, 0.5);
    double *g = gate ? arr(ng, &s, 0.05) : NULL, *h0 = with_h0 ? arr(ns, &s, 0.1) : NULL;
    double *o = arr(tv, &s, 0), *hT = arr(ns, &s, 0), *dout = arr(tv, &s, 1.0), *dhT = with_dhT ? arr(ns, &s, 1.0) : NULL;
    double *dq = arr(tk, &s, 0), *dkk = arr(tk, &s, 0), *dvv = arr(tv, &s, 0), *db = arr((size_t)BH * T, &s, 0);
    double *dg = gate ? arr(ng, &s, 0) : NULL, *dh0 = with_h0 ? arr(ns, &s, 0) : NULL;
    for (size_t i = 0; i < (size_t)BH * T; ++i) beta[i] = 0.5 + beta[i];
    for (size_t i = 0; i < ng; ++i) g[i] = -0.05 - g[i] * g[i];
    int rc = dn_oracle_fwd(BH, T, dk, dv, gate, q, k, v, beta, g, h0, o, hT, nthreads);
    rc |= dn_oracle_bwd(BH, T, dk, dv, gate, q, k, v, beta, g, h0, dout, dhT, dq, dkk, dvv, db, dg, dh0, nthreads);
    free(q); free(k); free(v); free(beta); free(g); free(h0); free(o); free(hT); free(dout); free(dhT);
    free(dq); free(dkk); free(dvv); free(db); free(dg); free(dh0);
    return rc;
}

int main(void)
{
    int bad = 0;
    for (int gate = 0; gate <= 2; ++gate) {
        bad |= run(2, 37, 8, 6, gate, 1, 1, 1);     /* ends inside the first checkpoint segment */
        bad |= run(3, 64 + 5, 4, 4, gate, 0, 0, 3); /* crosses a segment boundary, NULL h0 / dhT */
        bad |= run(1, 130, 16, 16, gate, 1, 0, 2);
        bad |= run(2, 1, 4, 8, gate, 1, 1, 4);      /* a single step, more threads than heads */
        bad |= run(1, 0, 4, 4, gate, 1, 1, 1);      /* no steps */
        bad |= run(0, 5, 4, 4, gate, 0, 0, 1);      /* no heads */
    }
    /* argument checks: these must fail cleanly */
    double x = 0;
    if (dn_oracle_fwd(1, 4, 0, 4, 0, &x, &x, &x, &x, NULL, NULL, &x, &x, 1) != -1) bad = 1;
    if (dn_oracle_fwd(1, 4, 4, 4, 1, &x, &x, &x, &x, NULL, NULL, &x, &x, 1) != -1) bad = 1;
    if (dn_oracle_bwd(1, 4, 4, 4, 0, &x, &x, &x, &x, NULL, NULL, &x, NULL, NULL, &x, &x, &x, NULL, NULL, 1) != -1) bad = 1;
    printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
    return bad;
}
