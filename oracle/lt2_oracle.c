/*
 * lt2_oracle.c -- plain fp64 CPU oracle of the LT2 gated-delta mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the HIP library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * library never does, and the two share no code, header or table.
 *
 * What it computes (LT2 explainer, paithon.it, section "Sostituire il
 * motore", the state-update equation):
 *
 *     S_t = A_t S_{t-1} + beta_t k_t v_t^T,
 *     A_t = Diag(alpha_t) (I - beta_t k_t k_t^T),
 *
 * with S_t a d_k x d_v matrix, k_t in R^{d_k}, v_t in R^{d_v}, beta_t a scalar
 * and alpha_t either one scalar per head (GDN) or one value per key channel
 * (KDA form; Diag(alpha_t) scales the rows of the state).  The pages give no
 * read-out; the one used is o_t = S_t^T q_t, taken after the update of token t,
 * with no scale.  Every (batch, head) unit runs its own recurrence.
 *
 * The update is applied exactly as written, one token at a time:
 *   (I - beta k k^T) S = S - beta k (k^T S)   (distributivity only), then the
 *   rows are scaled by alpha, then beta k v^T is added.  No chunking, no
 *   reordering across tokens, no intermediate rounding below fp64.
 *
 * Layouts (row-major, innermost last):
 *   q, k   [B, L, H, d_k]     v, o  [B, L, H, d_v]
 *   beta   [B, L, H]          alpha [B, L, H] (head gate) or [B, L, H, d_k]
 *   state  [B, H, d_k, d_v]
 */
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence on one unit's state S (d_k x d_v, row-major).
 * a points at alpha_t: one value (channel == 0) or d_k values (channel != 0).
 * kS is scratch of length d_v. */
static void gdn_token(int dk, int dv, int channel, const double *q, const double *k,
                      const double *v, const double *a, double beta, double *S,
                      double *o, double *kS)
{
    /* kS = S^T k  (the row vector k^T S) */
    for (int j = 0; j < dv; ++j) kS[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double ki = k[i];
        const double *Si = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) kS[j] += ki * Si[j];
    }
    /* S <- Diag(alpha) (S - beta k kS^T) + beta k v^T */
    for (int i = 0; i < dk; ++i) {
        const double ai = channel ? a[i] : a[0];
        const double bki = beta * k[i];
        double *Si = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) Si[j] = ai * (Si[j] - bki * kS[j]) + bki * v[j];
    }
    /* o = S^T q */
    if (o) {
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double qi = q[i];
            const double *Si = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) o[j] += qi * Si[j];
        }
    }
}

/*
 * Prefill: run the recurrence over L tokens for every (b, h) unit.
 *   S0    [B,H,d_k,d_v] initial state, or NULL for S_0 = 0
 *   o     [B,L,H,d_v] outputs (may be NULL)
 *   S_out [B,H,d_k,d_v] final state (may be NULL; may equal S0)
 *   nthreads <= 0 means the OpenMP default.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int lt2o_prefill(int B, int L, int H, int dk, int dv, int channel,
                 const double *q, const double *k, const double *v,
                 const double *alpha, const double *beta, const double *S0,
                 double *o, double *S_out, int nthreads)
{
    if (B < 0 || L < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !alpha || !beta) return -1;
    const long units = (long)B * H;
    const size_t sdim = (size_t)dk * dv;
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nthreads) reduction(| : err)
    {
        double *S = (double *)malloc(sizeof(double) * sdim);
        double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !kS) err = 1;
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!S || !kS) continue;
            const long b = u / H, h = u % H;
            if (S0) memcpy(S, S0 + (size_t)u * sdim, sizeof(double) * sdim);
            else memset(S, 0, sizeof(double) * sdim);
            for (long t = 0; t < L; ++t) {
                const size_t tok = (size_t)(b * L + t) * H + h;
                const double *a = channel ? alpha + tok * dk : alpha + tok;
                gdn_token(dk, dv, channel, q + tok * dk, k + tok * dk, v + tok * dv, a,
                          beta[tok], S, o ? o + tok * dv : NULL, kS);
            }
            if (S_out) memcpy(S_out + (size_t)u * sdim, S, sizeof(double) * sdim);
        }
        free(S);
        free(kS);
    }
    return err ? -1 : 0;
}

/*
 * Decode step: one token of the same recurrence for every (b, h) unit, state
 * updated in place.  q,k [B,H,d_k]; v,o [B,H,d_v]; beta [B,H];
 * alpha [B,H] or [B,H,d_k]; S [B,H,d_k,d_v].
 */
int lt2o_decode_step(int B, int H, int dk, int dv, int channel,
                     const double *q, const double *k, const double *v,
                     const double *alpha, const double *beta, double *S, double *o,
                     int nthreads)
{
    /* A decode step is a one-token prefill whose initial and final state are S. */
    return lt2o_prefill(B, 1, H, dk, dv, channel, q, k, v, alpha, beta, S, o, S, nthreads);
}

int lt2o_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
