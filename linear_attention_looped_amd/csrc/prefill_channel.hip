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
                                                           const float *__restrict__ state_in, TO *__restrict__ out,
                                                           float *__restrict__ state_out, int L, int H, int NC) {
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

size_t prefill_channel_ws_bytes(int B, int L, int H, int dk, int C) {
    const size_t NC = (size_t)((L + C - 1) / C);
    return (size_t)B * H * NC * ((size_t)4 * C * C + (size_t)C * dk + C) * sizeof(float);
}

namespace {

template <int D, int C, int PREC, typename TI, typename TO>
hipError_t run_channel(const GdnArgs &a, int phase, hipStream_t s) {
    constexpr int BV = 16;
    const int NC = (a.L + C - 1) / C;
    const unsigned units = (unsigned)a.B * (unsigned)a.H;
    if (phase & PHASE_PREPARE) {
        hipLaunchKernelGGL((prep_channel_kernel<D, C, PREC, TI>), dim3(units * NC), dim3(256), 0, s,
                           (const TI *)a.q, (const TI *)a.k, a.alpha, a.beta, (float *)a.ws, a.L, a.H, NC);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & PHASE_SCAN) {
        hipLaunchKernelGGL((scan_channel_kernel<D, D, BV, C, PREC, TI, TO>), dim3(units * (D / BV)), dim3(256), 0, s,
                           (const TI *)a.q, (const TI *)a.k, (const TI *)a.v, (const float *)a.ws,
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
