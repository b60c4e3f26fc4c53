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

/*
 * Backward pass (reverse-mode derivative) of lt2o_prefill for the scalar loss
 *     loss = sum_t <dO_t, o_t> + <dS_L, S_L>,
 * i.e. the vector-Jacobian product of the recurrence above with the output
 * cotangent dO and the final-state cotangent dS_L (NULL = 0).  Token by token
 * in reverse, with G the cotangent of the current state (after token t):
 *     G += q_t dO_t^T                 (o_t = S_t^T q_t)
 *     dq_t = S_t dO_t
 *     with P = S_{t-1} - beta k (k^T S_{t-1}) the undecayed erased state and
 *     G' = Diag(alpha_t) G:
 *     d(log alpha_t)  = alpha_t <G, P>          (head gate: summed over the state;
 *                       per channel i: alpha_ti sum_j G_ij P_ij)
 *     dv_t    = beta G^T k
 *     dbeta_t = k^T G v - k^T G' (S_{t-1}^T k)
 *     dk_t    = beta G v - beta (G' S_{t-1}^T k + S_{t-1} G'^T k)
 *     G      <- (I - beta k k^T) G'           (the cotangent of S_{t-1})
 * and finally dS_0 = G.  The states S_{t-1}, S_t are recomputed forward from
 * checkpoints kept every 64 tokens, one segment at a time (plain recomputation
 * of the same recurrence, not an approximation).  The gate gradient is taken
 * with respect to log alpha (finite at alpha = 0).
 * Outputs (all required): dq, dk [B,L,H,d_k]; dv [B,L,H,d_v]; dlog_alpha with
 * alpha's shape; dbeta [B,L,H]; dS0 [B,H,d_k,d_v].
 */
int lt2o_backward(int B, int L, int H, int dk, int dv, int channel,
                  const double *q, const double *k, const double *v,
                  const double *alpha, const double *beta, const double *S0,
                  const double *dO, const double *dSL,
                  double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                  double *dbeta, double *dS0, int nthreads)
{
    enum { SEG = 64 };
    if (B < 0 || L < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !alpha || !beta || !dO || !dq || !dk_out || !dv_out || !dlog_alpha || !dbeta || !dS0)
        return -1;
    const long units = (long)B * H;
    const size_t sdim = (size_t)dk * dv;
    const long nseg = (L + SEG - 1) / SEG;
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nthreads) reduction(| : err)
    {
        double *ck = (double *)malloc(sizeof(double) * sdim * (size_t)(nseg > 0 ? nseg : 1));
        double *Sb = (double *)malloc(sizeof(double) * sdim * (SEG + 1));
        double *G = (double *)malloc(sizeof(double) * sdim);
        double *Gp = (double *)malloc(sizeof(double) * sdim);
        double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
        double *gk = (double *)malloc(sizeof(double) * (size_t)dv);    /* G'^T k */
        if (!ck || !Sb || !G || !Gp || !kS || !gk) err = 1;
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (err) continue;
            const long b = u / H, h = u % H;
            /* forward: checkpoint the state before each segment */
            double *S = Sb;
            if (S0) memcpy(S, S0 + (size_t)u * sdim, sizeof(double) * sdim);
            else memset(S, 0, sizeof(double) * sdim);
            for (long t = 0; t < L; ++t) {
                if (t % SEG == 0) memcpy(ck + (size_t)(t / SEG) * sdim, S, sizeof(double) * sdim);
                const size_t tok = (size_t)(b * L + t) * H + h;
                const double *a = channel ? alpha + tok * dk : alpha + tok;
                gdn_token(dk, dv, channel, q + tok * dk, k + tok * dk, v + tok * dv, a, beta[tok], S, NULL, kS);
            }
            if (dSL) memcpy(G, dSL + (size_t)u * sdim, sizeof(double) * sdim);
            else memset(G, 0, sizeof(double) * sdim);
            for (long sg = nseg - 1; sg >= 0; --sg) {
                const long t0 = sg * SEG, t1 = (t0 + SEG < L) ? t0 + SEG : L;
                /* Sb[i] = state before token t0 + i, i = 0 .. t1 - t0 */
                memcpy(Sb, ck + (size_t)sg * sdim, sizeof(double) * sdim);
                for (long t = t0; t < t1; ++t) {
                    const size_t tok = (size_t)(b * L + t) * H + h;
                    const double *a = channel ? alpha + tok * dk : alpha + tok;
                    double *Sn = Sb + (size_t)(t - t0 + 1) * sdim;
                    memcpy(Sn, Sb + (size_t)(t - t0) * sdim, sizeof(double) * sdim);
                    gdn_token(dk, dv, channel, q + tok * dk, k + tok * dk, v + tok * dv, a, beta[tok], Sn, NULL, kS);
                }
                for (long t = t1 - 1; t >= t0; --t) {
                    const size_t tok = (size_t)(b * L + t) * H + h;
                    const double *qt = q + tok * dk, *kt = k + tok * dk, *vt = v + tok * dv;
                    const double *dot = dO + tok * dv;
                    const double *a = channel ? alpha + tok * dk : alpha + tok;
                    const double bt = beta[tok];
                    const double *Sp = Sb + (size_t)(t - t0) * sdim;      /* S_{t-1} */
                    const double *Sc = Sb + (size_t)(t - t0 + 1) * sdim;  /* S_t */
                    /* G += q dO^T ; dq = S_t dO */
                    for (int i = 0; i < dk; ++i) {
                        double acc = 0.0;
                        for (int j = 0; j < dv; ++j) {
                            G[(size_t)i * dv + j] += qt[i] * dot[j];
                            acc += Sc[(size_t)i * dv + j] * dot[j];
                        }
                        dq[tok * dk + i] = acc;
                    }
                    /* kS = S_{t-1}^T k */
                    for (int j = 0; j < dv; ++j) kS[j] = 0.0;
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) kS[j] += kt[i] * Sp[(size_t)i * dv + j];
                    /* gate gradient <G, P> (per row for the channel gate), G' = Diag(alpha) G */
                    double gsum = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        double ri = 0.0;
                        for (int j = 0; j < dv; ++j)
                            ri += G[(size_t)i * dv + j] * (Sp[(size_t)i * dv + j] - bt * kt[i] * kS[j]);
                        const double ai = channel ? a[i] : a[0];
                        if (channel) dlog_alpha[tok * dk + i] = ai * ri;
                        gsum += ri;
                        for (int j = 0; j < dv; ++j) Gp[(size_t)i * dv + j] = ai * G[(size_t)i * dv + j];
                    }
                    if (!channel) dlog_alpha[tok] = a[0] * gsum;
                    /* dv = beta G^T k ; gk = G'^T k */
                    for (int j = 0; j < dv; ++j) { dv_out[tok * dv + j] = 0.0; gk[j] = 0.0; }
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) {
                            dv_out[tok * dv + j] += bt * G[(size_t)i * dv + j] * kt[i];
                            gk[j] += Gp[(size_t)i * dv + j] * kt[i];
                        }
                    /* dbeta = k^T G v - k^T G' kS ; dk = beta G v - beta (G' kS + S_{t-1} gk) */
                    double db = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        double gv = 0.0, gks = 0.0, sgk = 0.0;
                        for (int j = 0; j < dv; ++j) {
                            gv += G[(size_t)i * dv + j] * vt[j];
                            gks += Gp[(size_t)i * dv + j] * kS[j];
                            sgk += Sp[(size_t)i * dv + j] * gk[j];
                        }
                        db += kt[i] * (gv - gks);
                        dk_out[tok * dk + i] = bt * gv - bt * (gks + sgk);
                    }
                    dbeta[tok] = db;
                    /* G <- (I - beta k k^T) G' */
                    for (int i = 0; i < dk; ++i) {
                        const double bki = bt * kt[i];
                        for (int j = 0; j < dv; ++j) G[(size_t)i * dv + j] = Gp[(size_t)i * dv + j] - bki * gk[j];
                    }
                }
            }
            memcpy(dS0 + (size_t)u * sdim, G, sizeof(double) * sdim);
        }
        free(ck); free(Sb); free(G); free(Gp); free(kS); free(gk);
    }
    return err ? -1 : 0;
}

int lt2o_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
