/* Drives the fp64 oracle (oracle/lt2_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: prefill, decode step and backward on small
 * seeded inputs, both gates, ragged lengths across the backward's 64-token
 * checkpoint segments, with and without initial states and state cotangents,
 * and the degenerate sizes.  Exit status 0 when every call succeeds and every
 * output is finite. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int lt2o_prefill(int B, int L, int H, int dk, int dv, int channel, const double *q, const double *k,
                 const double *v, const double *alpha, const double *beta, const double *S0, double *o,
                 double *S, int nthreads);
int lt2o_decode_step(int B, int H, int dk, int dv, int channel, const double *q, const double *k,
                     const double *v, const double *alpha, const double *beta, double *S, double *o,
                     int nthreads);
int lt2o_backward(int B, int L, int H, int dk, int dv, int channel, const double *q, const double *k,
                  const double *v, const double *alpha, const double *beta, const double *S0,
                  const double *dO, const double *dSL, double *dq, double *dk_out, double *dv_out,
                  double *dlog_alpha, double *dbeta, double *dS0, int nthreads);

static unsigned long long state = 88172645463325252ULL;
static double urand(void) {   /* xorshift64, uniform in [0, 1) */
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return (double)(state >> 11) * (1.0 / 9007199254740992.0);
}
static double *arr(size_t n, double lo, double hi) {
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
    return p;
}
static int finite_all(const double *p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int run(int B, int L, int H, int d, int channel, int with_state) {
    const size_t tok = (size_t)B * L * H, st = (size_t)B * H * d * d;
    double *q = arr(tok * d, -0.1, 0.1), *k = arr(tok * d, -0.1, 0.1), *v = arr(tok * d, -1, 1);
    double *al = arr(channel ? tok * d : tok, 0.0, 1.0), *be = arr(tok, 0.0, 1.0);
    double *S0 = with_state ? arr(st, -1, 1) : NULL, *dSL = with_state ? arr(st, -1, 1) : NULL;
    double *o = arr(tok * d, 0, 0), *S = arr(st, 0, 0), *dO = arr(tok * d, -1, 1);
    double *g[6];
    g[0] = arr(tok * d, 0, 0); g[1] = arr(tok * d, 0, 0); g[2] = arr(tok * d, 0, 0);
    g[3] = arr(channel ? tok * d : tok, 0, 0); g[4] = arr(tok, 0, 0); g[5] = arr(st, 0, 0);
    int bad = 0;
    bad |= lt2o_prefill(B, L, H, d, d, channel, q, k, v, al, be, S0, o, S, 2) != 0;
    bad |= !finite_all(o, tok * d) || !finite_all(S, st);
    bad |= lt2o_backward(B, L, H, d, d, channel, q, k, v, al, be, S0, dO, dSL, g[0], g[1], g[2], g[3], g[4], g[5],
                         2) != 0;
    bad |= !finite_all(g[0], tok * d) || !finite_all(g[3], channel ? tok * d : tok) || !finite_all(g[5], st);
    if (L > 0) {   /* one decode token on the prefill's final state (first token's inputs) */
        double *qd = arr((size_t)B * H * d, -0.1, 0.1), *od = arr((size_t)B * H * d, 0, 0);
        bad |= lt2o_decode_step(B, H, d, d, channel, qd, k, v, al, be, S, od, 1) != 0;
        bad |= !finite_all(od, (size_t)B * H * d);
        free(qd); free(od);
    }
    free(q); free(k); free(v); free(al); free(be); free(S0); free(dSL); free(o); free(S); free(dO);
    for (int i = 0; i < 6; ++i) free(g[i]);
    if (bad) fprintf(stderr, "failed: B=%d L=%d H=%d d=%d channel=%d state=%d\n", B, L, H, d, channel, with_state);
    return bad;
}

int main(void) {
    int bad = 0;
    const int Ls[] = {0, 1, 63, 64, 65, 130};
    for (int ch = 0; ch < 2; ++ch)
        for (int i = 0; i < 6; ++i)
            for (int ws = 0; ws < 2; ++ws) bad |= run(2, Ls[i], 2, 8, ch, ws);
    bad |= run(0, 10, 3, 8, 1, 1);
    bad |= run(1, 70, 1, 64, 1, 1);
    /* invalid arguments are refused */
    bad |= lt2o_prefill(-1, 4, 1, 8, 8, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) == 0;
    bad |= lt2o_backward(1, 4, 1, 8, 8, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                         NULL, NULL, 1) == 0;
    printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
    return bad;
}
