// prefill_channel.hip -- chunked prefill with one decay per key channel (KDA form).
//
// Recurrence with the ordering of the LT2 state-update equation (paithon.it,
// "Sostituire il motore"): S_t = Diag(a_t)(S_{t-1} - b_t k_t (k_t^T S_{t-1})) + b_t k_t v_t^T,
// a_t in R^{d_k}.  With e_t = -b_t S_{t-1}^T k_t each token is a rank-2 step
//   S_t = Diag(a_t) S_{t-1} + (a_t * k_t) e_t^T + b_t k_t v_t^T.
// Inside a chunk with state S entering it, g_t = sum_{j<=t} log2 a_j per channel
// (chunk-relative), gh_t = g_{t-1} (gh_0 = 0):
//   Ae_ti = b_t sum_c k_tc k_ic 2^(gh_tc - gh_ic)   (i < t)
//   Av_ti =     sum_c k_tc k_ic 2^(gh_tc - g_ic)    (i < t)
//   Pe_ti =     sum_c q_tc k_ic 2^(g_tc - gh_ic)    (i <= t)
//   Pv_ti = b_i sum_c q_tc k_ic 2^(g_tc - g_ic)     (i <= t)
//   Te = (I + Ae)^{-1} diag(b),  Nv = Te Av diag(b)
//   E  = -Te (K * 2^gh) S - Nv V
//   O  = (Q * 2^g) S + Pe E + Pv V
//   S <- 2^(g_C) * S + (K * 2^(g_C - gh))^T E + (b * K * 2^(g_C - g))^T V
// Every exponent above is <= 0.  The matrix-core form of the pairwise sums
// splits each factor through a reference point: for an off-diagonal 16-token
// block pair (rows in block I, columns in block J < I) the reference is g at
// the last token of block J, which keeps both factors <= 1 for any gate; for a
// diagonal block the reference is the per-channel midpoint of the block, used
// only while every channel's span inside the block stays below 240 (factors
// below 2^120); otherwise that block is summed pair by pair on the vector ALUs.
#include "common.h"
#include "internal.h"

namespace lt2 {

namespace {

constexpr float DIAG_SPAN_MAX = 240.f;   // log2 span allowed for the midpoint reference

// Workspace floats per chunk: Te, Nv, Pe, Pv [C][C], G [C][DK] and beta [C]
// (the scan phase takes its beta from here, not from the caller).
template <int DK, int C>
constexpr size_t chunk_floats() { return (size_t)4 * C * C + (size_t)C * DK + C; }

}  // namespace

// ---------------------------------------------------------------------------
// Prepare (chunk-parallel, 4 waves).
// ---------------------------------------------------------------------------
template <int DK, int C, int PREC, typename TI>
__global__ __launch_bounds__(256) void prep_channel_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                           const float *__restrict__ alpha,
                                                           const float *__restrict__ beta, float *__restrict__ ws,
                                                           int L, int H, int NC) {
    constexpr int GP = DK + 4;
    constexpr int CP = C + 4;
    constexpr int NT = C / 16;
    constexpr int NLT = NT * (NT + 1) / 2;
    constexpr int PARTS = 256 / DK;           // token segments of the per-channel prefix sum
    constexpr int SEG = C / PARTS;
    static_assert(256 % DK == 0 && C % PARTS == 0, "prefix layout");
    constexpr int G_BYTES = C * GP * 4, T_BYTES = C * CP * 4;
    __shared__ __attribute__((aligned(16))) unsigned char g_raw[G_BYTES > T_BYTES ? G_BYTES : T_BYTES];
    __shared__ float Am[C * CP];    // beta-scaled strict lower Ae
    __shared__ float Avm[C * CP];   // strict lower Av, later Av diag(beta)
    __shared__ float Xs[4][16 * 17];
    __shared__ float bs[C];
    __shared__ float seg_tot[PARTS][DK];
    float *G = reinterpret_cast<float *>(g_raw);   // g (base 2), later the inverse
    float *Ti = reinterpret_cast<float *>(g_raw);

    const int n = blockIdx.x % NC;
    const int unit = blockIdx.x / NC;
    const int h = unit % H, b = unit / H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const int t0 = n * C;
    const int Lc = min(C, L - t0);
    float *wsu = ws + ((size_t)unit * NC + n) * chunk_floats<DK, C>();
    float *Tg = wsu, *Ng = wsu + C * C, *Peg = wsu + 2 * C * C, *Pvg = wsu + 3 * C * C, *Gg = wsu + 4 * C * C;
    float *Bg = Gg + C * DK;
    const size_t tok0 = (size_t)b * L * H + h;   // token index of (b, t = 0, h) is tok0 + t*H

    // ---- per-channel prefix sums of log2(alpha) ----
    {
        const int c = tid % DK, p = tid / DK;
        float run = 0.f;
        for (int s = 0; s < SEG; ++s) {
            const int t = p * SEG + s;
            const float a = alpha[(tok0 + (size_t)(t0 + min(t, Lc - 1)) * H) * DK + c];
            run += (t < Lc) ? log2_gate(a) : 0.f;
            G[t * GP + c] = run;
        }
        seg_tot[p][c] = run;
    }
    if (tid < C) {
        const float bt = beta[tok0 + (size_t)(t0 + min(tid, Lc - 1)) * H];
        bs[tid] = (tid < Lc) ? bt : 0.f;
        Bg[tid] = (tid < Lc) ? bt : 0.f;
    }
    __syncthreads();
    {
        const int c = tid % DK, p = tid / DK;
        float off = 0.f;
        for (int pp = 0; pp < p; ++pp) off += seg_tot[pp][c];
        if (p > 0)
            for (int s = 0; s < SEG; ++s) G[(p * SEG + s) * GP + c] += off;
    }
    __syncthreads();
    for (int idx = tid; idx < C * DK / 4; idx += 256) {
        const int t = idx / (DK / 4), c4 = idx % (DK / 4);
        *reinterpret_cast<float4 *>(Gg + t * DK + 4 * c4) = *reinterpret_cast<const float4 *>(G + t * GP + 4 * c4);
    }

    // ---- pairwise gated sums, one 16x16 tile (I, J <= I) at a time per wave ----
    auto ghat = [&](int t, int c) { return t > 0 ? G[(t - 1) * GP + c] : 0.f; };
    for (int tt = wave; tt < NLT; tt += 4) {
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= tt) ++I;
        const int J = tt - I * (I + 1) / 2;
        const int trow = 16 * I + lr;   // A rows (t) and, as lane's B column, i = 16J + lr
        const int icol = 16 * J + lr;
        const TI *krow = k + (tok0 + (size_t)(t0 + min(trow, Lc - 1)) * H) * DK;
        const TI *qrow = q + (tok0 + (size_t)(t0 + min(trow, Lc - 1)) * H) * DK;
        const TI *kcol = k + (tok0 + (size_t)(t0 + min(icol, Lc - 1)) * H) * DK;
        const bool trow_ok = trow < Lc, icol_ok = icol < Lc;

        // references: off-diagonal -> g at the last token of block J; diagonal ->
        // per-channel midpoint of the block (guarded)
        bool use_mfma = true;
        if (I == J) {
            bool ok = true;
            for (int kb = 0; kb < DK / 32; ++kb)
                for (int e = 0; e < 8; ++e) {
                    const int c = 32 * kb + 8 * lq + e;
                    ok = ok && (ghat(16 * I, c) - G[(16 * I + 15) * GP + c] <= DIAG_SPAN_MAX);
                }
            use_mfma = __all(ok);
        }
        f32x4 ae = {0.f, 0.f, 0.f, 0.f}, av = ae, pe = ae, pv = ae;
        if (use_mfma) {
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag rk, rq, ck1, ck2, fk, fq, fkc;
                load_row8<TI>(fk, krow + 32 * kb + 8 * lq);
                load_row8<TI>(fq, qrow + 32 * kb + 8 * lq);
                load_row8<TI>(fkc, kcol + 32 * kb + 8 * lq);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = 32 * kb + 8 * lq + e;
                    const float ref = (I == J) ? 0.5f * (ghat(16 * I, c) + G[(16 * I + 15) * GP + c])
                                               : G[(16 * J + 15) * GP + c];
                    rk.x[e] = trow_ok ? fk.x[e] * exp2_fast(ghat(trow, c) - ref) : 0.f;
                    rq.x[e] = trow_ok ? fq.x[e] * exp2_fast(G[trow * GP + c] - ref) : 0.f;
                    ck1.x[e] = icol_ok ? fkc.x[e] * exp2_fast(ref - ghat(icol, c)) : 0.f;
                    ck2.x[e] = icol_ok ? fkc.x[e] * exp2_fast(ref - G[icol * GP + c]) : 0.f;
                }
                const auto ork = make_op<PREC, false>(rk), orq = make_op<PREC, false>(rq);
                const auto oc1 = make_op<PREC, false>(ck1), oc2 = make_op<PREC, false>(ck2);
                mma_op<PREC, false, false>(ae, ork, oc1);
                mma_op<PREC, false, false>(av, ork, oc2);
                mma_op<PREC, false, false>(pe, orq, oc1);
                mma_op<PREC, false, false>(pv, orq, oc2);
            }
        } else {
            // exact pairwise sums (diagonal block whose gate span is too large)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + 4 * lq + r, i = 16 * J + lr;
                if (i > t || t >= Lc) continue;
                const TI *kt = k + (tok0 + (size_t)(t0 + t) * H) * DK;
                const TI *qt = q + (tok0 + (size_t)(t0 + t) * H) * DK;
                const TI *ki = k + (tok0 + (size_t)(t0 + i) * H) * DK;
                float s1 = 0.f, s2 = 0.f, s3 = 0.f, s4 = 0.f;
                for (int c = 0; c < DK; ++c) {
                    const float kk = load1<TI>(kt + c) * load1<TI>(ki + c);
                    const float qk = load1<TI>(qt + c) * load1<TI>(ki + c);
                    const float gt = G[t * GP + c], gi = G[i * GP + c];
                    const float ght = ghat(t, c), ghi = ghat(i, c);
                    if (i < t) {
                        s1 += kk * exp2_fast(ght - ghi);
                        s2 += kk * exp2_fast(ght - gi);
                    }
                    s3 += qk * exp2_fast(gt - ghi);
                    s4 += qk * exp2_fast(gt - gi);
                }
                ae[r] = s1; av[r] = s2; pe[r] = s3; pv[r] = s4;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + 4 * lq + r, i = 16 * J + lr;
            Am[t * CP + i] = (i < t) ? bs[t] * ae[r] : 0.f;
            Avm[t * CP + i] = (i < t) ? av[r] * bs[i] : 0.f;
            Peg[t * C + i] = (i <= t && t < Lc) ? pe[r] : 0.f;
            Pvg[t * C + i] = (i <= t && t < Lc) ? pv[r] * bs[i] : 0.f;
        }
    }
    // zero the upper tiles of the workspace outputs and of Am / Avm
    for (int tt = wave; tt < NT * NT; tt += 4) {
        const int I = tt / NT, J = tt % NT;
        if (J <= I) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + 4 * lq + r, i = 16 * J + lr;
            Am[t * CP + i] = 0.f;
            Avm[t * CP + i] = 0.f;
            Peg[t * C + i] = 0.f;
            Pvg[t * C + i] = 0.f;
        }
    }
    __syncthreads();   // G is dead from here on: its space becomes the inverse

    // ---- (I + Ae)^{-1}: diagonal blocks by forward substitution, then by distance ----
    if (wave < NT && lane < 16) {
        const int base = 16 * wave;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float s = (t == lane) ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < t; ++s2) s -= Am[(base + t) * CP + base + s2] * x[s2];
            x[t] = s;
        }
        for (int t = 0; t < C; ++t) Ti[t * CP + base + lane] = (t >= base && t < base + 16) ? x[t - base] : 0.f;
    }
    __syncthreads();
    for (int dist = 1; dist < NT; ++dist) {
        if (wave < NT - dist) {
            const int J = wave, I = wave + dist;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int Kb = J; Kb < I; ++Kb) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float a = Am[(16 * I + lr) * CP + 16 * Kb + 4 * kk + lq];
                    const float bb = Ti[(16 * Kb + 4 * kk + lq) * CP + 16 * J + lr];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Xs[wave][(4 * lq + r) * 17 + lr] = acc[r];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float a = Ti[(16 * I + lr) * CP + 16 * I + 4 * kk + lq];
                const float bb = Xs[wave][(4 * kk + lq) * 17 + lr];
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, y, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Ti[(16 * I + 4 * lq + r) * CP + 16 * J + lr] = -y[r];
        }
        __syncthreads();
    }

    // ---- Te = T diag(beta) (into Am), then Nv = Te (Av diag(beta)) ----
    for (int idx = tid; idx < C * C; idx += 256) {
        const int t = idx / C, i = idx % C;
        const float te = (i <= t) ? Ti[t * CP + i] * bs[i] : 0.f;
        Am[t * CP + i] = te;
        Tg[idx] = te;
    }
    __syncthreads();
    for (int tt = wave; tt < NT * NT; tt += 4) {
        const int I = tt / NT, J = tt % NT;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (J < I || J == I) {
            for (int Kb = J; Kb <= I; ++Kb) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float a = Am[(16 * I + lr) * CP + 16 * Kb + 4 * kk + lq];
                    const float bb = Avm[(16 * Kb + 4 * kk + lq) * CP + 16 * J + lr];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Ng[(16 * I + 4 * lq + r) * C + 16 * J + lr] = acc[r];
    }
}

// ---------------------------------------------------------------------------
// Scan (sequential over chunks) for one (b, h, BV-column block), 4 waves.
// Wave w owns output row tile w (C = 64) and state tiles w, w + 4 (d_k = 128).
// ---------------------------------------------------------------------------
template <int DK, int DV, int BV, int C, int PREC, typename TI, typename TO>
__global__ __launch_bounds__(256) void scan_channel_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                           const TI *__restrict__ v, const float *__restrict__ ws,
                                                           const float *state_in, TO *__restrict__ out,
                                                           float *state_out, int L, int H, int NC) {
    constexpr int KP = DK + 4;
    constexpr int CP = C + 4;
    constexpr int NTR = C / 16, NTK = DK / 16;
    constexpr int NTV = BV / 16;
    constexpr int NT_O = NTR * NTV, NT_S = NTK * NTV;
    constexpr int MAXO = (NT_O + 3) / 4, MAXS = (NT_S + 3) / 4;
    constexpr int NKB_C = (C + 31) / 32;
    constexpr int NV = DV / BV;
    static_assert(4 % NTR == 0, "a wave's output tiles share one row tile");
    static_assert(4 % NTV == 0 && NT_S % 4 == 0, "a wave's state tiles share one column tile");

    __shared__ __attribute__((aligned(16))) float Kg[C * KP];      // K * 2^gh
    __shared__ __attribute__((aligned(16))) float K1T[DK * CP];    // (K * 2^(gC - gh))^T
    __shared__ __attribute__((aligned(16))) float K2T[DK * CP];    // (b K * 2^(gC - g))^T
    __shared__ __attribute__((aligned(16))) float St[BV * KP];     // S^T
    __shared__ __attribute__((aligned(16))) float Xt[BV * CP], Vt[BV * CP], Et[BV * CP];
    __shared__ float gC[DK];

    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    const int vb = logical % NV;
    const size_t unit = logical / NV;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const int v0 = vb * BV;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const int I = wave % NTR;
    const bool has_o = wave < NT_O;
    const int nkb = (16 * I + 16 + 31) / 32;
    const int Js = wave % NTV;
    const size_t tok0 = (size_t)b * L * H + h;

    f32x4 Sacc[MAXS];
#pragma unroll
    for (int m = 0; m < MAXS; ++m) {
        const int Ik = (wave + 4 * m) / NTV;
        Sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (state_in) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sacc[m][r] = state_in[(unit * DK + 16 * Ik + 4 * lq + r) * DV + v0 + 16 * Js + lr];
        }
        *reinterpret_cast<float4 *>(St + (16 * Js + lr) * KP + 16 * Ik + 4 * lq) =
            make_float4(Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
    }

    for (int n = 0; n < NC; ++n) {
        const int t0 = n * C;
        const int Lc = min(C, L - t0);
        const float *wsu = ws + (unit * NC + n) * chunk_floats<DK, C>();
        const float *Tg = wsu, *Ng = wsu + C * C, *Peg = wsu + 2 * C * C, *Pvg = wsu + 3 * C * C;
        const float *Gg = wsu + 4 * C * C;
        const float *Bg = Gg + C * DK;
        __syncthreads();
        // gate-scaled copies of K: K*2^gh (rows), (K*2^(gC-gh))^T, (b K*2^(gC-g))^T
        for (int idx = tid; idx < C * DK; idx += 256) {
            const int t = idx / DK, c = idx % DK;
            const int tc = min(t, Lc - 1);
            const float kv = (t < Lc) ? load1<TI>(k + (tok0 + (size_t)(t0 + tc) * H) * DK + c) : 0.f;
            const float bt = Bg[t];   // zero past the ragged end
            const float g = Gg[t * DK + c];
            const float gh = t > 0 ? Gg[(t - 1) * DK + c] : 0.f;
            const float gc = Gg[(Lc - 1) * DK + c];
            Kg[t * KP + c] = kv * exp2_fast(gh);
            K1T[c * CP + t] = kv * exp2_fast(gc - gh);
            K2T[c * CP + t] = bt * kv * exp2_fast(gc - g);
            if (t == 0) gC[c] = gc;
        }
        for (int idx = tid; idx < C * BV; idx += 256) {
            const int t = idx / BV, j = idx % BV;
            const float vv = (t < Lc) ? load1<TI>(v + (tok0 + (size_t)(t0 + min(t, Lc - 1)) * H) * DV + v0 + j) : 0.f;
            Vt[j * CP + t] = vv;
        }
        __syncthreads();

        // X = (K*2^gh) S -> Xt;  O = (Q*2^g) S (registers)
        f32x4 Oacc[MAXO];
#pragma unroll
        for (int m = 0; m < MAXO; ++m) Oacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (has_o) {
            const int trow = 16 * I + lr;
            const bool tok = trow < Lc;
            const TI *qrow = q + (tok0 + (size_t)(t0 + min(trow, Lc - 1)) * H) * DK;
            f32x4 xk[MAXO];
#pragma unroll
            for (int m = 0; m < MAXO; ++m) xk[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag fk, fq;
                load_frag_f32(fk, Kg + trow * KP + 32 * kb + 8 * lq);
                load_row8<TI>(fq, qrow + 32 * kb + 8 * lq);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    fq.x[e] = tok ? fq.x[e] * exp2_fast(Gg[trow * DK + 32 * kb + 8 * lq + e]) : 0.f;
                const auto ak = make_op<PREC, false>(fk);
                const auto aq = make_op<PREC, false>(fq);
#pragma unroll
                for (int m = 0; m < MAXO; ++m) {
                    const int o = wave + 4 * m;
                    if (o >= NT_O) continue;
                    const int J = o / NTR;
                    Frag fs;
                    load_frag_f32(fs, St + (16 * J + lr) * KP + 32 * kb + 8 * lq);
                    const auto bs = make_op<PREC, false>(fs);
                    mma_op<PREC, false, false>(xk[m], ak, bs);
                    mma_op<PREC, false, false>(Oacc[m], aq, bs);
                }
            }
#pragma unroll
            for (int m = 0; m < MAXO; ++m) {
                const int o = wave + 4 * m;
                if (o >= NT_O) continue;
                const int J = o / NTR;
                *reinterpret_cast<float4 *>(Xt + (16 * J + lr) * CP + 16 * I + 4 * lq) =
                    make_float4(xk[m][0], xk[m][1], xk[m][2], xk[m][3]);
            }
        }
        __syncthreads();

        // E = -(Te X + Nv V) -> Et
        if (has_o) {
#pragma unroll
            for (int m = 0; m < MAXO; ++m) {
                const int o = wave + 4 * m;
                if (o >= NT_O) continue;
                const int J = o / NTR;
                f32x4 ea = {0.f, 0.f, 0.f, 0.f};
                for (int kb = 0; kb < nkb; ++kb) {
                    const int kc = min(32 * kb + 8 * lq, C - 8);
                    const bool kin = 32 * kb + 8 * lq < C;
                    Frag ft, fn, fx, fv;
                    load_frag_f32(ft, Tg + (16 * I + lr) * C + kc);
                    load_frag_f32(fn, Ng + (16 * I + lr) * C + kc);
                    load_frag_f32(fx, Xt + (16 * J + lr) * CP + kc);
                    load_frag_f32(fv, Vt + (16 * J + lr) * CP + kc);
                    if (!kin) { zero_frag(ft); zero_frag(fn); }
                    mma_op<PREC, false, false>(ea, make_op<PREC, false>(ft), make_op<PREC, false>(fx));
                    mma_op<PREC, false, (PREC == PREC_BF16) && sizeof(TI) == 2>(ea, make_op<PREC, false>(fn),
                        make_op<PREC, (PREC == PREC_BF16) && sizeof(TI) == 2>(fv));
                }
                *reinterpret_cast<float4 *>(Et + (16 * J + lr) * CP + 16 * I + 4 * lq) =
                    make_float4(-ea[0], -ea[1], -ea[2], -ea[3]);
            }
        }
        __syncthreads();

        // O += Pe E + Pv V, store
        if (has_o) {
#pragma unroll
            for (int m = 0; m < MAXO; ++m) {
                const int o = wave + 4 * m;
                if (o >= NT_O) continue;
                const int J = o / NTR;
                for (int kb = 0; kb < nkb; ++kb) {
                    const int kc = min(32 * kb + 8 * lq, C - 8);
                    const bool kin = 32 * kb + 8 * lq < C;
                    Frag fp, fq, fe, fv;
                    load_frag_f32(fp, Peg + (16 * I + lr) * C + kc);
                    load_frag_f32(fq, Pvg + (16 * I + lr) * C + kc);
                    load_frag_f32(fe, Et + (16 * J + lr) * CP + kc);
                    load_frag_f32(fv, Vt + (16 * J + lr) * CP + kc);
                    if (!kin) { zero_frag(fp); zero_frag(fq); }
                    mma_op<PREC, false, false>(Oacc[m], make_op<PREC, false>(fp), make_op<PREC, false>(fe));
                    mma_op<PREC, false, (PREC == PREC_BF16) && sizeof(TI) == 2>(Oacc[m], make_op<PREC, false>(fq),
                        make_op<PREC, (PREC == PREC_BF16) && sizeof(TI) == 2>(fv));
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * I + 4 * lq + r;
                    if (t < Lc) store1<TO>(out + (tok0 + (size_t)(t0 + t) * H) * DV + v0 + 16 * J + lr, Oacc[m][r]);
                }
            }
        }

        // S <- 2^gC * S + K1^T E + K2^T V
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
            const int Ik = (wave + 4 * m) / NTV;
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[m][r] *= exp2_fast(gC[16 * Ik + 4 * lq + r]);
        }
#pragma unroll
        for (int kb = 0; kb < NKB_C; ++kb) {
            const int kc = min(32 * kb + 8 * lq, C - 8);
            const bool kin = 32 * kb + 8 * lq < C;
            Frag fe, fv;
            load_frag_f32(fe, Et + (16 * Js + lr) * CP + kc);
            load_frag_f32(fv, Vt + (16 * Js + lr) * CP + kc);
            if (!kin) { zero_frag(fe); zero_frag(fv); }
            const auto be = make_op<PREC, false>(fe);
            const auto bv = make_op<PREC, (PREC == PREC_BF16) && sizeof(TI) == 2>(fv);
#pragma unroll
            for (int m = 0; m < MAXS; ++m) {
                const int Ik = (wave + 4 * m) / NTV;
                Frag f1, f2;
                load_frag_f32(f1, K1T + (16 * Ik + lr) * CP + kc);
                load_frag_f32(f2, K2T + (16 * Ik + lr) * CP + kc);
                mma_op<PREC, false, false>(Sacc[m], make_op<PREC, false>(f1), be);
                mma_op<PREC, false, (PREC == PREC_BF16) && sizeof(TI) == 2>(Sacc[m], make_op<PREC, false>(f2), bv);
            }
        }
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
            const int Ik = (wave + 4 * m) / NTV;
            *reinterpret_cast<float4 *>(St + (16 * Js + lr) * KP + 16 * Ik + 4 * lq) =
                make_float4(Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
        }
    }

    if (state_out) {
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
            const int Ik = (wave + 4 * m) / NTV;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                state_out[(unit * DK + 16 * Ik + 4 * lq + r) * DV + v0 + 16 * Js + lr] = Sacc[m][r];
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 inputs: transition form of a chunk.
// Substituting E into the output and state updates above gives, for the state
// S entering a chunk,
//   O  = Qt S + Pt V,   Qt = Q * 2^g - Pe Te (K * 2^gh),   Pt = Pv - Pe Nv
//   S' = M S  + N V,    M  = diag(2^gC) - K1^T Te (K * 2^gh),  N = K2^T - K1^T Nv
// with K1 = K * 2^(gC - gh), K2 = b K * 2^(gC - g) and Nv = Te Av diag(b).  With
// Z = K1^T Te and PT = Pe Te the whole (DK + C) x (DK + CK) matrix is
//   W = [[M, N], [Qt, Pt]] = [[diag(2^gC), K2^T], [Q * 2^g, Pv]] - [Z; PT] [K * 2^gh | Av diag(b)]
// (CK = C rounded up to a whole K-block of 32, the extra columns zero).  The
// prepare phase forms W per chunk; the scan then does one product per chunk,
// [S'; O] = W [S; V], with no dependency chain inside the chunk.
//
// W is stored as MFMA A-fragments in bf16 hi/lo: 16-row tile R, K-block kb,
// hi then lo, 64 lanes x 16 bytes.  Lane (r, q) (r = lane % 16, q = lane / 16)
// holds W[16R + r][32kb + 4q + s] in slot s < 4 and W[16R + r][32kb + 16 + 4q + s - 4]
// in slots 4..7: the column order of two accumulator tiles of W^T, which the
// scan matches by reading its B operand in the same order.
// ---------------------------------------------------------------------------
namespace {

template <int DK, int C>
struct TmShape {
    static constexpr int CK = C < 32 ? 32 : C;       // token extent in whole K-blocks
    static constexpr int NRR = (DK + C) / 16;        // 16-row tiles of W
    static constexpr int NKW = (DK + CK) / 32;       // K-blocks of W
    static constexpr size_t BYTES = (size_t)NRR * NKW * 2048;   // per chunk
};

}  // namespace

template <int DK, int C>
__global__ __launch_bounds__(512) void prep_channel_tm_kernel(const uint16_t *__restrict__ q,
                                                              const uint16_t *__restrict__ k,
                                                              const float *__restrict__ alpha,
                                                              const float *__restrict__ beta,
                                                              unsigned char *__restrict__ ws, int L, int H, int NC) {
    using SH = TmShape<DK, C>;
    constexpr int NTH = 512, NW = 8;
    constexpr int GP = DK + 4;    // fp32 pitch of G rows
    constexpr int CP = C + 4;     // fp32 pitch of C-wide matrices
    constexpr int KTP = C + 8;    // bf16 pitch of K^T rows
    constexpr int NT = C / 16;
    constexpr int NLT = NT * (NT + 1) / 2;
    constexpr int PARTS = NTH / DK;
    constexpr int SEG = C / PARTS;
    constexpr int CK = SH::CK, NKW = SH::NKW, NRR = SH::NRR;
    constexpr int NKT = CK / 32;                      // K-blocks over tokens
    constexpr int ZR = DK > C ? DK : C;               // rows of the inverse / Z buffer
    constexpr bool XS_IN_TZ = (DK - C) * CP >= 4 * 16 * 17;   // distance-loop scratch fits above the inverse
    static_assert(NTH % DK == 0 && C % PARTS == 0 && SEG >= 1, "prefix layout");

    __shared__ __attribute__((aligned(16))) float G[C * GP];          // g (base 2, chunk-relative)
    __shared__ __attribute__((aligned(16))) uint16_t KT[DK * KTP];     // K^T, zero past the ragged end
    __shared__ __attribute__((aligned(16))) float Am[C * CP];         // b-scaled Ae, then Te
    __shared__ __attribute__((aligned(16))) float Avm[C * CP];        // Av diag(b)
    __shared__ __attribute__((aligned(16))) float Pem[C * CP];        // Pe, then PT = Pe Te
    __shared__ __attribute__((aligned(16))) float Pvm[C * CP];        // Pv (b-scaled columns)
    __shared__ __attribute__((aligned(16))) float TZ[ZR * CP];        // inverse T, then Z = K1^T Te
    __shared__ float Xs_own[XS_IN_TZ ? 1 : 4 * 16 * 17];
    constexpr int QP = DK + 8;                        // bf16 pitch of the staged Q rows
    constexpr bool QS_IN_AM = DK <= 2 * C;            // Q fits where Te was once Te is no longer read
    __shared__ __attribute__((aligned(16))) uint16_t Qs_own[QS_IN_AM ? 8 : C * QP];
    __shared__ float bs[C];
    __shared__ float seg_tot[PARTS][DK];
    float *Xs = XS_IN_TZ ? TZ + C * CP : Xs_own;

    const int n = blockIdx.x % NC;
    const int unit = blockIdx.x / NC;
    const int h = unit % H, b = unit / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    const int t0 = n * C;
    const int Lc = min(C, L - t0);
    const size_t tok0 = (size_t)b * L * H + h;   // token index of (b, t = 0, h) is tok0 + t*H
    unsigned char *wsu = ws + ((size_t)unit * NC + n) * SH::BYTES;

    // ---- K^T (bf16), beta, per-channel prefix sums of log2(alpha) ----
    // (all global loads of this step are issued before any of them is used)
    // K pieces are token-major across lanes, so the transposed LDS writes of a
    // wave land in consecutive banks.
    constexpr int KPT = (C * DK / 8 + NTH - 1) / NTH;
    uint4 kraw[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = min(tid + NTH * i, C * DK / 8 - 1);
        const int t = idx % C, c0 = 8 * (idx / C);
        kraw[i] = *reinterpret_cast<const uint4 *>(k + (tok0 + (size_t)(t0 + min(t, Lc - 1)) * H) * DK + c0);
    }
    const int pc = tid % DK, pp0 = tid / DK;   // prefix-sum roles: channel, token segment
    float alph[SEG];
#pragma unroll
    for (int s2 = 0; s2 < SEG; ++s2)
        alph[s2] = alpha[(tok0 + (size_t)(t0 + min(pp0 * SEG + s2, Lc - 1)) * H) * DK + pc];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = tid + NTH * i;
        if (idx < C * DK / 8) {
            const int t = idx % C, c0 = 8 * (idx / C);
            const uint4 u = (t < Lc) ? kraw[i] : make_uint4(0u, 0u, 0u, 0u);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                KT[(c0 + 2 * e) * KTP + t] = (uint16_t)(w[e] & 0xFFFFu);
                KT[(c0 + 2 * e + 1) * KTP + t] = (uint16_t)(w[e] >> 16);
            }
        }
    }
    {
        float run = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < SEG; ++s2) {
            const int t = pp0 * SEG + s2;
            const float lg = materialize(log2_gate(alph[s2]));   // every lane, then selected
            run += (t < Lc) ? lg : 0.f;
            G[t * GP + pc] = run;
        }
        seg_tot[pp0][pc] = run;
    }
    if (tid < C) {
        const float bt = beta[tok0 + (size_t)(t0 + min(tid, Lc - 1)) * H];
        bs[tid] = (tid < Lc) ? bt : 0.f;
    }
    __syncthreads();
    {
        const int c = tid % DK, p = tid / DK;
        float off = 0.f;
        for (int pp = 0; pp < p; ++pp) off += seg_tot[pp][c];
        if (p > 0)
            for (int s2 = 0; s2 < SEG; ++s2) G[(p * SEG + s2) * GP + c] += off;
    }
    __syncthreads();

    // ---- pairwise gated sums, one 16x16 tile (I, J <= I) at a time per wave ----
    // g_{t-1} (zero at t = 0): the load is issued for every lane, then selected
    auto ghat = [&](int t, int c) {
        const float x = materialize(G[max(t - 1, 0) * GP + c]);
        return t > 0 ? x : 0.f;
    };
    for (int tt = wave; tt < NLT; tt += NW) {
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= tt) ++I;
        const int J = tt - I * (I + 1) / 2;
        const int trow = 16 * I + lr;
        const int icol = 16 * J + lr;
        const uint16_t *krow = k + (tok0 + (size_t)(t0 + min(trow, Lc - 1)) * H) * DK;
        const uint16_t *qrow = q + (tok0 + (size_t)(t0 + min(trow, Lc - 1)) * H) * DK;
        const uint16_t *kcol = k + (tok0 + (size_t)(t0 + min(icol, Lc - 1)) * H) * DK;
        const bool trow_ok = trow < Lc, icol_ok = icol < Lc;
        // eight consecutive channels of a G row (row -1 reads as zeros)
        auto grow8 = [&](Frag &f, int row, int c0) {
            load_frag_f32(f, G + max(row, 0) * GP + c0);
            const bool z = row < 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) f.x[e] = z ? 0.f : f.x[e];
        };
        bool use_mfma = true;
        if (I == J) {
            bool ok = true;
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag a, z;
                grow8(a, 16 * I - 1, 32 * kb + 8 * lq);
                grow8(z, 16 * I + 15, 32 * kb + 8 * lq);
#pragma unroll
                for (int e = 0; e < 8; ++e) ok &= (a.x[e] - z.x[e] <= DIAG_SPAN_MAX);
            }
            use_mfma = __all(ok);
        }
        f32x4 ae = {0.f, 0.f, 0.f, 0.f}, av = ae, pe = ae, pv = ae;
        if (use_mfma) {
            Raw8<uint16_t> rk8[DK / 32], rq8[DK / 32], rc8[DK / 32];
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                load_raw8<uint16_t>(rk8[kb], krow + 32 * kb + 8 * lq);
                load_raw8<uint16_t>(rq8[kb], qrow + 32 * kb + 8 * lq);
                load_raw8<uint16_t>(rc8[kb], kcol + 32 * kb + 8 * lq);
            }
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                const int c0 = 32 * kb + 8 * lq;
                Frag rk, rq, ck1, ck2, fk, fq, fkc, gt, ght, gi, ghi, ref;
                raw_to_frag(fk, rk8[kb]);
                raw_to_frag(fq, rq8[kb]);
                raw_to_frag(fkc, rc8[kb]);
                grow8(gt, trow, c0);
                grow8(ght, trow - 1, c0);
                grow8(gi, icol, c0);
                grow8(ghi, icol - 1, c0);
                if (I == J) {
                    Frag a, z;
                    grow8(a, 16 * I - 1, c0);
                    grow8(z, 16 * I + 15, c0);
#pragma unroll
                    for (int e = 0; e < 8; ++e) ref.x[e] = 0.5f * (a.x[e] + z.x[e]);
                } else {
                    grow8(ref, 16 * J + 15, c0);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // computed for every lane, then selected (see materialize)
                    const float xk = materialize(fk.x[e] * exp2_fast(ght.x[e] - ref.x[e]));
                    const float xq = materialize(fq.x[e] * exp2_fast(gt.x[e] - ref.x[e]));
                    const float xc1 = materialize(fkc.x[e] * exp2_fast(ref.x[e] - ghi.x[e]));
                    const float xc2 = materialize(fkc.x[e] * exp2_fast(ref.x[e] - gi.x[e]));
                    rk.x[e] = trow_ok ? xk : 0.f;
                    rq.x[e] = trow_ok ? xq : 0.f;
                    ck1.x[e] = icol_ok ? xc1 : 0.f;
                    ck2.x[e] = icol_ok ? xc2 : 0.f;
                }
                const auto ork = make_op<PREC_BF16, false>(rk), orq = make_op<PREC_BF16, false>(rq);
                const auto oc1 = make_op<PREC_BF16, false>(ck1), oc2 = make_op<PREC_BF16, false>(ck2);
                mma_op<PREC_BF16, false, false>(ae, ork, oc1);
                mma_op<PREC_BF16, false, false>(av, ork, oc2);
                mma_op<PREC_BF16, false, false>(pe, orq, oc1);
                mma_op<PREC_BF16, false, false>(pv, orq, oc2);
            }
        } else {
            // exact pairwise sums (diagonal block whose gate span is too large)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + 4 * lq + r, i = 16 * J + lr;
                if (i > t || t >= Lc) continue;
                const uint16_t *kt = k + (tok0 + (size_t)(t0 + t) * H) * DK;
                const uint16_t *qt = q + (tok0 + (size_t)(t0 + t) * H) * DK;
                const uint16_t *ki = k + (tok0 + (size_t)(t0 + i) * H) * DK;
                float s1 = 0.f, s2 = 0.f, s3 = 0.f, s4 = 0.f;
                for (int c = 0; c < DK; ++c) {
                    const float kk = bf16_to_f32(kt[c]) * bf16_to_f32(ki[c]);
                    const float qk = bf16_to_f32(qt[c]) * bf16_to_f32(ki[c]);
                    const float gt = G[t * GP + c], gi = G[i * GP + c];
                    const float ght = ghat(t, c), ghi = ghat(i, c);
                    if (i < t) {
                        s1 += kk * exp2_fast(ght - ghi);
                        s2 += kk * exp2_fast(ght - gi);
                    }
                    s3 += qk * exp2_fast(gt - ghi);
                    s4 += qk * exp2_fast(gt - gi);
                }
                ae[r] = s1; av[r] = s2; pe[r] = s3; pv[r] = s4;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + 4 * lq + r, i = 16 * J + lr;
            const float bt = materialize(bs[t]), bi = materialize(bs[i]);   // every lane, then selected
            Am[t * CP + i] = (i < t) ? bt * ae[r] : 0.f;
            Avm[t * CP + i] = (i < t) ? av[r] * bi : 0.f;
            Pem[t * CP + i] = (i <= t && t < Lc) ? pe[r] : 0.f;
            Pvm[t * CP + i] = (i <= t && t < Lc) ? pv[r] * bi : 0.f;
        }
    }
    for (int tt = wave; tt < NT * NT; tt += NW) {   // upper tiles
        const int I = tt / NT, J = tt % NT;
        if (J <= I) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + 4 * lq + r, i = 16 * J + lr;
            Am[t * CP + i] = 0.f;
            Avm[t * CP + i] = 0.f;
            Pem[t * CP + i] = 0.f;
            Pvm[t * CP + i] = 0.f;
        }
    }
    __syncthreads();

    // ---- T = (I + Ae)^{-1}: diagonal blocks by forward substitution, then by distance ----
    float *Ti = TZ;
    if (wave < NT && lane < 16) {
        const int base = 16 * wave;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float s2 = (t == lane) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < t; ++j) s2 -= Am[(base + t) * CP + base + j] * x[j];
            x[t] = s2;
        }
        // rows of the block from registers (static indices), zeros elsewhere in its columns
#pragma unroll
        for (int t = 0; t < 16; ++t) Ti[(base + t) * CP + base + lane] = x[t];
        for (int t = 0; t < C; ++t)
            if (t < base || t >= base + 16) Ti[t * CP + base + lane] = 0.f;
    }
    __syncthreads();
    for (int dist = 1; dist < NT; ++dist) {
        if (wave < NT - dist) {
            const int J = wave, I = wave + dist;
            float *X = Xs + wave * 16 * 17;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int Kb = J; Kb < I; ++Kb) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float a = Am[(16 * I + lr) * CP + 16 * Kb + 4 * kk + lq];
                    const float bb = Ti[(16 * Kb + 4 * kk + lq) * CP + 16 * J + lr];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) X[(4 * lq + r) * 17 + lr] = acc[r];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float a = Ti[(16 * I + lr) * CP + 16 * I + 4 * kk + lq];
                const float bb = X[(4 * kk + lq) * 17 + lr];
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, y, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Ti[(16 * I + 4 * lq + r) * CP + 16 * J + lr] = -y[r];
        }
        __syncthreads();
    }
    // Te = T diag(b), into Am
    for (int idx = tid; idx < C * C; idx += NTH) {
        const int t = idx / C, i = idx % C;
        const float x = materialize(Ti[t * CP + i] * bs[i]);   // every element, then selected
        Am[t * CP + i] = (i <= t) ? x : 0.f;
    }
    __syncthreads();

    // Fragments over a token K-block kt: Te (B operand, rows = tokens) and the
    // gate-scaled K^T rows (A operand).  Tokens past C (C < 32) are zero.
    auto te_frag = [&](Frag &f, int kt, int col) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = 32 * kt + 8 * lq + e;
            f.x[e] = (C >= 32 || i < C) ? Am[i * CP + col] : 0.f;   // C >= 32: every token in range
        }
    };

    // Q rows for the W^T step, loaded now and staged once Te is no longer read
    constexpr int QPT = (C * DK / 8 + NTH - 1) / NTH;
    uint4 qraw[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int idx = min(tid + NTH * i, C * DK / 8 - 1);
        const int t = idx / (DK / 8), c0 = 8 * (idx % (DK / 8));
        qraw[i] = *reinterpret_cast<const uint4 *>(q + (tok0 + (size_t)(t0 + min(t, Lc - 1)) * H) * DK + c0);
    }

    // ---- Z = K1^T Te (DK x C, into TZ) and PT = Pe Te (C x C, in place of Pe) ----
    constexpr int ZT = (DK / 16) * NT;
    for (int tt = wave; tt < ZT + NT; tt += NW) {
        if (tt < ZT) {
            const int Rz = tt / NT, Jz = tt % NT;
            const int c = 16 * Rz + lr;
            const float gc = G[(C - 1) * GP + c];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                Frag a, bfr;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int i = 32 * kt + 8 * lq + e;
                    a.x[e] = (C >= 32 || i < C) ? bf16_to_f32(KT[c * KTP + i]) * exp2_fast(gc - ghat(i, c)) : 0.f;
                }
                te_frag(bfr, kt, 16 * Jz + lr);
                mma<PREC_BF16, false, false>(acc, a, bfr);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) TZ[(16 * Rz + 4 * lq + r) * CP + 16 * Jz + lr] = acc[r];
        } else {
            const int I = tt - ZT;   // this wave alone reads and rewrites rows I of Pe
            f32x4 acc[NT];
#pragma unroll
            for (int J = 0; J < NT; ++J) {
                acc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    Frag a, bfr;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int i = 32 * kt + 8 * lq + e;
                        a.x[e] = (C >= 32 || i < C) ? Pem[(16 * I + lr) * CP + i] : 0.f;
                    }
                    te_frag(bfr, kt, 16 * J + lr);
                    mma<PREC_BF16, false, false>(acc[J], a, bfr);
                }
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int J = 0; J < NT; ++J) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Pem[(16 * I + 4 * lq + r) * CP + 16 * J + lr] = acc[J][r];
            }
        }
    }
    __syncthreads();

    uint16_t *Qs = QS_IN_AM ? reinterpret_cast<uint16_t *>(Am) : Qs_own;
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int idx = tid + NTH * i;
        if (idx < C * DK / 8) {
            const int t = idx / (DK / 8), c0 = 8 * (idx % (DK / 8));
            *reinterpret_cast<uint4 *>(&Qs[t * QP + c0]) = (t < Lc) ? qraw[i] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __syncthreads();

    // ---- W^T tiles -> A-fragments of W, hi/lo ----
    // Task = (K-block kb of W, group of row tiles R): the A operand of W^T for
    // the two 16-column tiles 2kb, 2kb + 1 ([K * 2^gh | Av diag(b)]^T rows) is
    // built once and reused for every R of the group.
    constexpr int RG = 4, RPG = (NRR + RG - 1) / RG;
    for (int task = wave; task < NKW * RG; task += NW) {
        const int kb = task % NKW, rg = task / NKW;
        bf16x8 ah[2][NKT], al[2][NKT];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int T = 2 * kb + half;   // 16-column tile of W (uniform)
            const int w = 16 * T + lr;     // A row: a W column
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const int j0 = 32 * kt + 8 * lq;   // first of this lane's eight tokens
                Frag a;
                zero_frag(a);
                if (C >= 32 || j0 < C) {   // C >= 32: every token in range
                    if (16 * T < DK) {          // (K * 2^gh)^T
                        const uint4 u = *reinterpret_cast<const uint4 *>(&KT[w * KTP + j0]);
                        Raw8<uint16_t> r8;
                        r8.u = u;
                        raw_to_frag(a, r8);
#pragma unroll
                        for (int e = 0; e < 8; ++e) a.x[e] *= exp2_fast(ghat(j0 + e, w));
                    } else if (16 * T < DK + C) {   // (Av diag(b))^T
#pragma unroll
                        for (int e = 0; e < 8; ++e) a.x[e] = Avm[(j0 + e) * CP + (w - DK)];
                    }
                }
                split_bf16(a, ah[half][kt], al[half][kt]);
            }
        }
        for (int R = rg * RPG; R < min(NRR, (rg + 1) * RPG); ++R) {
            const int r = 16 * R + lr;     // this lane's W row (B column)
            const bool srow = R < DK / 16; // state rows (M, N) or output rows (Qt, Pt); uniform
            const float *brow = srow ? TZ + r * CP : Pem + (r - DK) * CP;
            bf16x8 bh[NKT], bl[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                Frag bfr;
                if (C >= 32 || 32 * kt + 8 * lq + 8 <= C) load_frag_f32(bfr, brow + 32 * kt + 8 * lq);
                else zero_frag(bfr);
                split_bf16(bfr, bh[kt], bl[kt]);
            }
            const float gcr = srow ? G[(C - 1) * GP + r] : 0.f;
            float vals[8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int T = 2 * kb + half;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (16 * T < DK + C) {
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt) {
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[half][kt], bh[kt], acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[half][kt], bh[kt], acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[half][kt], bl[kt], acc, 0, 0, 0);
                    }
                }
                // base at W[r][w], w = 16T + 4lq + e (the block is uniform per (R, T))
                const int w0 = 16 * T + 4 * lq;
                float base[4] = {0.f, 0.f, 0.f, 0.f};
                if (srow) {
                    if (16 * T < DK) {                    // diag(2^gC)
#pragma unroll
                        for (int e = 0; e < 4; ++e) base[e] = (w0 + e == r) ? exp2_fast(gcr) : 0.f;
                    } else if (16 * T < DK + C) {         // K2^T = (b K * 2^(gC - g))^T
                        const int i0 = w0 - DK;
                        const uint2 u = *reinterpret_cast<const uint2 *>(&KT[r * KTP + i0]);
                        const float kk[4] = {__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                                             __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            base[e] = bs[i0 + e] * kk[e] * exp2_fast(gcr - G[(i0 + e) * GP + r]);
                    }
                } else {
                    const int t = r - DK;
                    if (16 * T < DK) {                    // Q * 2^g
                        const uint2 u = *reinterpret_cast<const uint2 *>(&Qs[t * QP + w0]);
                        const float4 g4 = *reinterpret_cast<const float4 *>(&G[t * GP + w0]);
                        base[0] = __uint_as_float(u.x << 16) * exp2_fast(g4.x);
                        base[1] = __uint_as_float(u.x & 0xFFFF0000u) * exp2_fast(g4.y);
                        base[2] = __uint_as_float(u.y << 16) * exp2_fast(g4.z);
                        base[3] = __uint_as_float(u.y & 0xFFFF0000u) * exp2_fast(g4.w);
                    } else if (16 * T < DK + C) {         // Pv
                        const float4 p4 = *reinterpret_cast<const float4 *>(&Pvm[t * CP + (w0 - DK)]);
                        base[0] = p4.x; base[1] = p4.y; base[2] = p4.z; base[3] = p4.w;
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) vals[4 * half + e] = base[e] - acc[e];
            }
            uint4 hi, lo;
            split8(vals, hi, lo);
            unsigned char *dst = wsu + (size_t)(R * NKW + kb) * 2048 + 16 * lane;
            // W streams to HBM (2.4 GB on a 32k-token, 32-head prefill) and is read
            // back only by the scan: non-temporal stores (prepare 2.37 -> 2.30 ms
            // on that workload)
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, hi), reinterpret_cast<u32x4 *>(dst));
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, lo), reinterpret_cast<u32x4 *>(dst + 1024));
        }
    }
}

// Scan in transition form for one (b, h, 16-column block of V), 8 waves:
// [S'; O] = W [S; V] per chunk.  Wave w owns state rows 16w..16w+15 (w < DK/16)
// and one half of the K-blocks of output row tile w % 4 (first half for
// w < 4); the two halves are summed when the staged outputs are stored.
// A-fragments of W go from the workspace straight into registers, one chunk
// ahead, the same number of loads in every wave (a wave without a role loads a
// valid tile and skips its products); S^T (hi/lo) and V^T are read from LDS in
// the fragments' permuted column order.
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

template <int DK, int C>
struct TmFrags {   // one chunk's A-fragments of this wave (hi, lo per K-block)
    static constexpr int NKW = TmShape<DK, C>::NKW;
    static constexpr int NKH = (NKW + 1) / 2;
    u32x4 s[NKW][2];   // state rows: all K-blocks (S part, then V part)
    u32x4 o[NKH][2];   // output rows: this wave's half of the K-blocks
};

template <int DK, int DV, int C, typename TO>
__global__ __launch_bounds__(512) void scan_channel_tm_kernel(const uint16_t *__restrict__ v,
                                                              const unsigned char *__restrict__ ws,
                                                              const float *state_in,
                                                              TO *__restrict__ out, float *state_out,
                                                              int L, int H, int NC) {
    using SH = TmShape<DK, C>;
    using FR = TmFrags<DK, C>;
    constexpr int NW = 8, BV = 16;
    constexpr int CK = SH::CK, NKW = SH::NKW;
    constexpr int NKS = DK / 32, NKV = CK / 32;
    constexpr int SP = DK + 8;              // bf16 pitch of S^T rows
    constexpr int VP = CK + 8;              // bf16 pitch of V^T rows
    constexpr int OP = BV + 4;              // fp32 pitch of the output halves
    constexpr int NTR = C / 16;
    constexpr int OV = 16 / (int)sizeof(TO);
    constexpr int NO = C * BV / OV;         // 16-byte output pieces per chunk
    constexpr int NVP = C * BV / 8;         // 16-byte V pieces per chunk
    constexpr int NV = DV / BV;
    static_assert(NTR <= 4 && DK / 16 <= NW && NO <= 512 && NVP <= 512, "scan roles");

    __shared__ __attribute__((aligned(16))) uint16_t Sth[2][BV * SP], Stl[2][BV * SP];
    __shared__ __attribute__((aligned(16))) uint16_t VT[2][BV * VP];
    __shared__ __attribute__((aligned(16))) float Oh[2][2][C * OP];

    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    const int vb = logical % NV;
    const size_t unit = logical / NV;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const int v0 = vb * BV;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    constexpr int NKH = FR::NKH;
    const bool has_s = DK / 16 == NW || wave < DK / 16;
    const int oI = wave & 3, oh = wave >> 2;               // output row tile, K-block half
    const bool has_o = NTR == 4 || oI < NTR;
    const unsigned vtok_stride = (unsigned)H * DV;
    const uint16_t *vb_ptr = v + ((size_t)b * L * H + h) * DV + v0;
    TO *ob_ptr = out + ((size_t)b * L * H + h) * DV + v0;
    const size_t lane_off = 16 * (size_t)lane;

    auto frag_addr = [&](int n, int R, int kb) __attribute__((always_inline)) {
        return ws + (unit * NC + (unsigned)n) * SH::BYTES + (size_t)(R * NKW + kb) * 2048 + lane_off;
    };
    const int Rs = min(wave, DK / 16 - 1);           // state row tile (valid for every wave)
    const int Ro = DK / 16 + min(oI, NTR - 1);        // output row tile of W
    auto fetch = [&](int n, FR &f) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < NKW; ++kb) {
            const unsigned char *p = frag_addr(n, Rs, kb);
            f.s[kb][0] = *reinterpret_cast<const u32x4 *>(p);
            f.s[kb][1] = *reinterpret_cast<const u32x4 *>(p + 1024);
        }
#pragma unroll
        for (int j = 0; j < NKH; ++j) {
            const unsigned char *p = frag_addr(n, Ro, min(oh * NKH + j, NKW - 1));
            f.o[j][0] = *reinterpret_cast<const u32x4 *>(p);
            f.o[j][1] = *reinterpret_cast<const u32x4 *>(p + 1024);
        }
    };
    // V pieces: token row vrow, columns vcol..vcol+7 of this block
    const int vidx = min(tid, NVP - 1);
    const int vrow = vidx / (BV / 8), vcol = 8 * (vidx % (BV / 8));
    auto fetch_v = [&](int n) __attribute__((always_inline)) {
        u32x4 r = {0u, 0u, 0u, 0u};
        const int last = min(C, L - n * C) - 1;
        if (NVP % 64 == 0 ? wave < NVP / 64 : tid < NVP)
            r = *reinterpret_cast<const u32x4 *>(vb_ptr + (size_t)n * C * vtok_stride +
                                                 (unsigned)min(vrow, last) * vtok_stride + (unsigned)vcol);
        return r;
    };
    auto stage_v = [&](const u32x4 &r, int buf) __attribute__((always_inline)) {
        if (NVP % 64 == 0 ? wave < NVP / 64 : tid < NVP) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                VT[buf][(vcol + 2 * e) * VP + vrow] = (uint16_t)(r[e] & 0xFFFFu);
                VT[buf][(vcol + 2 * e + 1) * VP + vrow] = (uint16_t)(r[e] >> 16);
            }
        }
    };
    // B fragments in the permuted column order: slots 0..3 = rows 32kb + 4lq + 0..3,
    // slots 4..7 = rows 32kb + 16 + 4lq + 0..3 of S (resp. V)
    auto bfrag = [&](const uint16_t *rowp, int kb) __attribute__((always_inline)) {
        const u32x2 x0 = *reinterpret_cast<const u32x2 *>(rowp + 32 * kb + 4 * lq);
        const u32x2 x1 = *reinterpret_cast<const u32x2 *>(rowp + 32 * kb + 16 + 4 * lq);
        return __builtin_bit_cast(bf16x8, u32x4{x0[0], x0[1], x1[0], x1[1]});
    };
    auto store_o = [&](int n, int rows, int buf) __attribute__((always_inline)) {   // outputs of chunk n
        const int oidx = min(tid, NO - 1);
        const int orow = oidx / (BV / OV), ocol = OV * (oidx % (BV / OV));
        if ((NO % 64 == 0 ? wave < NO / 64 : tid < NO) && orow < rows) {
            float x[OV];
#pragma unroll
            for (int e = 0; e < OV; ++e) x[e] = Oh[buf][0][orow * OP + ocol + e] + Oh[buf][1][orow * OP + ocol + e];
            TO *dst = ob_ptr + ((size_t)n * C + orow) * vtok_stride + ocol;
            if constexpr (sizeof(TO) == 2) {
                uint4 hi, lo;
                split8(x, hi, lo);
                *reinterpret_cast<uint4 *>(dst) = hi;
            } else {
                *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
            }
        }
    };

    // initial state -> S^T[0]; chunk 0's fragments and V
    f32x4 Sacc = {0.f, 0.f, 0.f, 0.f};
    if (has_s) {
        if (state_in) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[r] = state_in[(unit * DK + 16 * wave + 4 * lq + r) * DV + v0 + lr];
        }
        const float x[4] = {Sacc[0], Sacc[1], Sacc[2], Sacc[3]};
        uint2 h2, l2;
        split4(x, h2, l2);
        *reinterpret_cast<uint2 *>(&Sth[0][lr * SP + 16 * wave + 4 * lq]) = h2;
        *reinterpret_cast<uint2 *>(&Stl[0][lr * SP + 16 * wave + 4 * lq]) = l2;
    }
    if (CK > C) {   // V^T columns past the chunk stay zero
        for (int idx = tid; idx < 2 * BV * VP; idx += 512) (&VT[0][0])[idx] = 0;
        __syncthreads();
    }
    stage_v(fetch_v(0), 0);
    FR pa, pb;
    fetch(0, pa);

    // L2 prefetch two chunks ahead: the NV column-block workgroups of a unit each
    // touch one in NV of that chunk's 128-byte workspace lines with a 4-byte
    // load, so the fragments fetched into registers a chunk later come from L2
    // rather than HBM (the scan is otherwise bound by that fetch's latency).  The
    // loaded word is only passed to an empty asm one chunk later, so nothing
    // waits for it in between.
    constexpr int LINES = (int)(SH::BYTES / 128), PFL = (LINES + NV - 1) / NV;
    unsigned pf_word = 0u;
    auto prefetch_l2 = [&](int n) __attribute__((always_inline)) {
        asm volatile("" ::"v"(pf_word));   // the previous prefetch has landed by now
        const int line = vb * PFL + tid;
        if (n < NC && tid < PFL && line < LINES)
            pf_word = *reinterpret_cast<const unsigned *>(ws + (unit * NC + (unsigned)n) * SH::BYTES +
                                                          (size_t)line * 128);
    };

    auto chunk = [&](int n, FR &cur, FR &nxt) __attribute__((always_inline)) {
        const int buf = n & 1;
        __syncthreads();   // S^T, V^T of chunk n and the outputs of chunk n - 1 are in LDS
        const int nn = min(n + 1, NC - 1);   // the last chunk re-fetches itself (unused)
        fetch(nn, nxt);
        prefetch_l2(n + 2);
        const u32x4 vn = fetch_v(nn);
        if (n > 0) store_o(n - 1, C, buf ^ 1);

        const uint16_t *sh = &Sth[buf][lr * SP], *sl = &Stl[buf][lr * SP], *vt = &VT[buf][lr * VP];
        if (has_s) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKS; ++kb) {
                const bf16x8 ah = __builtin_bit_cast(bf16x8, cur.s[kb][0]);
                const bf16x8 al = __builtin_bit_cast(bf16x8, cur.s[kb][1]);
                const bf16x8 bh = bfrag(sh, kb), bl = bfrag(sl, kb);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
            }
#pragma unroll
            for (int kb = 0; kb < NKV; ++kb) {
                const bf16x8 ah = __builtin_bit_cast(bf16x8, cur.s[NKS + kb][0]);
                const bf16x8 al = __builtin_bit_cast(bf16x8, cur.s[NKS + kb][1]);
                const bf16x8 bv = bfrag(vt, kb);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, acc, 0, 0, 0);
            }
            Sacc = acc;
        }
        if (has_o) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NKH; ++j) {
                const int kb = oh * NKH + j;   // wave-uniform
                const bf16x8 ah = __builtin_bit_cast(bf16x8, cur.o[j][0]);
                const bf16x8 al = __builtin_bit_cast(bf16x8, cur.o[j][1]);
                if (kb < NKS) {
                    const bf16x8 bh = bfrag(sh, kb), bl = bfrag(sl, kb);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
                } else if (kb < NKW) {
                    const bf16x8 bv = bfrag(vt, kb - NKS);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Oh[buf][oh][(16 * oI + 4 * lq + r) * OP + lr] = acc[r];
        }
        if (has_s) {
            const float x[4] = {Sacc[0], Sacc[1], Sacc[2], Sacc[3]};
            uint2 h2, l2;
            split4(x, h2, l2);
            *reinterpret_cast<uint2 *>(&Sth[buf ^ 1][lr * SP + 16 * wave + 4 * lq]) = h2;
            *reinterpret_cast<uint2 *>(&Stl[buf ^ 1][lr * SP + 16 * wave + 4 * lq]) = l2;
        }
        stage_v(vn, buf ^ 1);
    };
    int n = 0;
    for (; n + 1 < NC; n += 2) {
        chunk(n, pa, pb);
        chunk(n + 1, pb, pa);
    }
    if (n < NC) chunk(n, pa, pb);
    __syncthreads();
    store_o(NC - 1, L - (NC - 1) * C, (NC - 1) & 1);

    if (state_out && has_s) {
#pragma unroll
        for (int r = 0; r < 4; ++r) state_out[(unit * DK + 16 * wave + 4 * lq + r) * DV + v0 + lr] = Sacc[r];
    }
}

size_t prefill_channel_ws_bytes(int B, int L, int H, int dk, int C, bool bf16) {
    const size_t NC = (size_t)((L + C - 1) / C);
    if (bf16) {
        const size_t CK = C < 32 ? 32 : C;
        return (size_t)B * H * NC * (size_t)(dk + C) * (dk + CK) * 4;
    }
    return (size_t)B * H * NC * ((size_t)4 * C * C + (size_t)C * dk + C) * sizeof(float);
}

namespace {

template <int D, int C, int PREC, typename TI, typename TO>
hipError_t run_channel(const GdnArgs &a, int phase, hipStream_t s) {
    constexpr int BV = 16;
    const int NC = (a.L + C - 1) / C;
    const unsigned units = (unsigned)a.B * (unsigned)a.H;
    if (phase & PHASE_PREPARE) {
        if constexpr (PREC == PREC_BF16)
            hipLaunchKernelGGL((prep_channel_tm_kernel<D, C>), dim3(units * NC), dim3(512), 0, s,
                               (const uint16_t *)a.q, (const uint16_t *)a.k, a.alpha, a.beta,
                               (unsigned char *)a.ws, a.L, a.H, NC);
        else
            hipLaunchKernelGGL((prep_channel_kernel<D, C, PREC, TI>), dim3(units * NC), dim3(256), 0, s,
                               (const TI *)a.q, (const TI *)a.k, a.alpha, a.beta, (float *)a.ws, a.L, a.H, NC);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & PHASE_SCAN) {
        if constexpr (PREC == PREC_BF16)
            hipLaunchKernelGGL((scan_channel_tm_kernel<D, D, C, TO>), dim3(units * (D / BV)), dim3(512), 0, s,
                               (const uint16_t *)a.v, (const unsigned char *)a.ws, a.state_in, (TO *)a.out,
                               a.state_out, a.L, a.H, NC);
        else
            hipLaunchKernelGGL((scan_channel_kernel<D, D, BV, C, PREC, TI, TO>), dim3(units * (D / BV)), dim3(256), 0,
                               s, (const TI *)a.q, (const TI *)a.k, (const TI *)a.v, (const float *)a.ws,
                               a.state_in, (TO *)a.out, a.state_out, a.L, a.H, NC);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int D, int C>
hipError_t run_channel_t(const GdnArgs &a, int phase, hipStream_t s) {
    if (a.qkv_bf16)
        return a.out_bf16 ? run_channel<D, C, PREC_BF16, uint16_t, uint16_t>(a, phase, s)
                          : run_channel<D, C, PREC_BF16, uint16_t, float>(a, phase, s);
    return a.out_bf16 ? run_channel<D, C, PREC_F32, float, uint16_t>(a, phase, s)
                      : run_channel<D, C, PREC_F32, float, float>(a, phase, s);
}

template <int D>
hipError_t run_channel_c(const GdnArgs &a, int phase, hipStream_t s) {
    switch (a.chunk) {
        case 16: return run_channel_t<D, 16>(a, phase, s);
        case 32: return run_channel_t<D, 32>(a, phase, s);
        default: return run_channel_t<D, 64>(a, phase, s);
    }
}

}  // namespace

hipError_t launch_prefill_channel(const GdnArgs &a, int phase, hipStream_t s) {
    return a.dk == 64 ? run_channel_c<64>(a, phase, s) : run_channel_c<128>(a, phase, s);
}

}  // namespace lt2
