// prefill_head.hip -- chunked prefill of the gated delta rule, one decay per head.
//
// Recurrence (LT2 explainer, paithon.it, "Sostituire il motore"):
//   S_t = a_t (S_{t-1} - b_t k_t k_t^T S_{t-1}) + b_t k_t v_t^T,  o_t = S_t^T q_t.
// Writing u_t = b_t (v_t - a_t S_{t-1}^T k_t) gives S_t = a_t S_{t-1} + k_t u_t^T.
// Inside a chunk of C tokens with state S entering it, g_t = sum_{j<=t} log a_j
// (chunk-relative) and Gamma_ti = exp(g_t - g_i):
//   (I + A) U = diag(b) (V - diag(e^g) K S),   A_ti = b_t Gamma_ti k_t.k_i  (i < t)
//   U = Tm (V - diag(e^g) K S),                Tm = (I + A)^{-1} diag(b)
//   O = diag(e^g) Q S + P U,                   P_ti = Gamma_ti q_t.k_i      (i <= t)
//   S <- e^{g_C} S + K^T diag(e^{g_C - g}) U
// Tm and P do not depend on the state: the prepare kernel forms them for every
// chunk in parallel; the scan kernel carries the fp32 state across the chunks
// of one unit in order, for one block of BV state columns (columns evolve
// independently), with the next chunk's inputs in flight while the current
// chunk computes.
//
// Gate exponents are masked before exp, so every exponent is <= 0.
#include "common.h"
#include "internal.h"

namespace lt2 {

// ---------------------------------------------------------------------------
// Prepare: per chunk, Tm = (I + A)^{-1} diag(beta), P and the gate prefix g
// (base 2).  Workspace per (b, h, chunk), 8*C*C + 12*C bytes:
//   fp32 inputs: Tm [C][C] f32 | P [C][C] f32 | g, 2^g, 2^(g_C - g) [C] f32
//   bf16 inputs: Tm hi, Tm lo, P hi, P lo [C][C] bf16 | g, 2^g, 2^(g_C - g) [C] f32
// (hi = bf16(x), lo = bf16(x - hi): the scan feeds them to bf16 matrix cores
// without converting).  Tm and P are zero above the diagonal.
// ---------------------------------------------------------------------------
// One 32-wide k block of a product of two input fragments (eight consecutive
// elements per lane, the common.h fragment layout).  bf16 inputs on the bf16
// path go to the matrix core as they are; otherwise through fp32 fragments.
template <int PREC, typename TI>
__device__ __forceinline__ void gram_mma(f32x4 &acc, const Raw8<TI> &a, const Raw8<TI> &b) {
    if constexpr (PREC == PREC_BF16 && sizeof(TI) == 2) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                      0, 0, 0);
    } else {
        Frag fa, fb;
        raw_to_frag(fa, a);
        raw_to_frag(fb, b);
        mma<PREC, true, true>(acc, fa, fb);
    }
}

template <int DK, int C, int PREC, typename TI>
__global__ __launch_bounds__(256) void prep_head_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                        const float *__restrict__ alpha,
                                                        const float *__restrict__ beta,
                                                        unsigned char *__restrict__ ws, int L, int H, int NC) {
    constexpr int KP = DK + 16 / (int)sizeof(TI);   // row pitch (elements), rows stay 16-byte aligned
    constexpr int CP = C + 4;
    constexpr int NT = C / 16;
    constexpr int NLT = NT * (NT + 1) / 2;           // lower tiles (incl. diagonal)
    constexpr int MAXP = (NLT + 3) / 4;              // Q K^T tiles per wave
    constexpr int K_BYTES = C * KP * (int)sizeof(TI);
    constexpr int T_BYTES = C * CP * 4;
    // K is dead once the Gram tiles are formed; the inverse reuses its space.
    __shared__ __attribute__((aligned(16))) unsigned char kt_raw[K_BYTES > T_BYTES ? K_BYTES : T_BYTES];
    __shared__ float Am[C * CP];   // gated K K^T, then P
    __shared__ float Xs[4][16 * 17];
    __shared__ float bs[C];
    __shared__ double gs[C];   // fp64: see the gate-prefix comment below
    TI *Ks = reinterpret_cast<TI *>(kt_raw);
    float *Ti = reinterpret_cast<float *>(kt_raw);

    const int n = blockIdx.x % NC;
    const int unit = blockIdx.x / NC;
    const int h = unit % H, b = unit / H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const int t0 = n * C;
    const int Lc = min(C, L - t0);
    unsigned char *wsu = ws + ((size_t)unit * NC + n) * (size_t)(8 * C * C + 12 * C);
    float *gg = reinterpret_cast<float *>(wsu + 8 * C * C);

    // Q fragments of this wave's Q K^T tiles, fetched together with K so that
    // the global latency is paid once
    Raw8<TI> qraw[MAXP][DK / 32];
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
        const int tt = min(wave + 4 * m, NLT - 1);
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= tt) ++I;
        const int arow = 16 * I + lr;
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
            load_raw8<TI>(qraw[m][kb], q + ((size_t)(b * (size_t)L + t0 + min(arow, Lc - 1)) * H + h) * DK + 32 * kb + 8 * lq);
    }
    constexpr int KPT = (C * (DK / 8) + 255) / 256;
    Raw8<TI> kraw[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = min(tid + 256 * i, C * (DK / 8) - 1);
        const int t = idx / (DK / 8), c8 = idx % (DK / 8);
        load_raw8<TI>(kraw[i], k + ((size_t)(b * (size_t)L + t0 + min(t, Lc - 1)) * H + h) * DK + 8 * c8);
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = tid + 256 * i;
        if (idx < C * (DK / 8)) {
            const int t = idx / (DK / 8), c8 = idx % (DK / 8);
            if (t >= Lc) zero_raw8<TI>(kraw[i]);
            *reinterpret_cast<Raw8<TI> *>(Ks + t * KP + 8 * c8) = kraw[i];
        }
    }
    if (wave == 0) {
        const size_t tok = (size_t)(b * (size_t)L + t0 + min(lane, Lc - 1)) * H + h;
        const float a_raw = alpha[tok], b_raw = beta[tok];
        // chunk-relative prefix of log2 alpha in fp64: a fast decay reaches hundreds
        // of octaves within a chunk, where an fp32 sum would give every decay
        // 2^(g_t - g_i) between nearby tokens a relative error of |g| 2^-24
        double lg = (lane < Lc) ? (double)log2_gate(a_raw) : 0.0;
        const float bt = (lane < Lc) ? b_raw : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(lg, off);
            if (lane >= off) lg += y;
        }
        if (lane < C) { gs[lane] = lg; bs[lane] = bt; }
    }
    __syncthreads();

    // Gated K K^T (strictly lower, rows scaled by beta) into Am; gated Q K^T
    // tiles (lower incl.) stay in registers until the inverse is done.
    for (int tt = wave; tt < NT * NT; tt += 4) {
        const int I = tt / NT, J = tt % NT;
        if (J > I) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Am[(16 * I + 4 * lq + r) * CP + 16 * J + lr] = 0.f;
            continue;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
            gram_mma<PREC>(acc, *reinterpret_cast<const Raw8<TI> *>(Ks + (16 * I + lr) * KP + 32 * kb + 8 * lq),
                           *reinterpret_cast<const Raw8<TI> *>(Ks + (16 * J + lr) * KP + 32 * kb + 8 * lq));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + 4 * lq + r, i = 16 * J + lr;
            Am[t * CP + i] = (i < t) ? bs[t] * exp2_fast((float)(gs[t] - gs[i])) * acc[r] : 0.f;
        }
    }
    f32x4 pacc[MAXP];
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
        pacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tt = wave + 4 * m;
        if (tt >= NLT) continue;
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= tt) ++I;
        const int J = tt - I * (I + 1) / 2;
        const int arow = 16 * I + lr;
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            Raw8<TI> qa = qraw[m][kb];
            if (arow >= Lc) zero_raw8<TI>(qa);
            gram_mma<PREC>(pacc[m], qa, *reinterpret_cast<const Raw8<TI> *>(Ks + (16 * J + lr) * KP + 32 * kb + 8 * lq));
        }
    }
    __syncthreads();

    // (I + A)^{-1}: 16x16 diagonal blocks by forward substitution (one wave per
    // block, lane j < 16 solves column j) ...
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
#pragma unroll
        for (int t = 0; t < 16; ++t) Ti[(base + t) * CP + base + lane] = x[t];
    }
    __syncthreads();
    // ... then the blocks below the diagonal by distance:
    //   T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ   (fp32 matrix cores)
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

    // Gated P into Am's space (Am is dead after the inverse), zero above the diagonal.
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
        const int tt = wave + 4 * m;
        if (tt >= NLT) continue;
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= tt) ++I;
        const int J = tt - I * (I + 1) / 2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + 4 * lq + r, i = 16 * J + lr;
            Am[t * CP + i] = (i <= t && t < Lc) ? exp2_fast((float)(gs[t] - gs[i])) * pacc[m][r] : 0.f;
        }
    }
    for (int tt = wave; tt < NT * NT; tt += 4) {
        const int I = tt / NT, J = tt % NT;
        if (J <= I) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) Am[(16 * I + 4 * lq + r) * CP + 16 * J + lr] = 0.f;
    }
    __syncthreads();

    // Coalesced stores: eight consecutive entries per lane.  Tm = T diag(beta).
    for (int idx = tid; idx < C * C / 8; idx += 256) {
        const int t = idx / (C / 8), i0 = 8 * (idx % (C / 8));
        float tv[8], pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            tv[e] = (i0 + e <= t) ? Ti[t * CP + i0 + e] * bs[i0 + e] : 0.f;
            pv[e] = Am[t * CP + i0 + e];
        }
        if constexpr (PREC == PREC_F32) {
            float *Tg = reinterpret_cast<float *>(wsu), *Pg = Tg + C * C;
            *reinterpret_cast<float4 *>(Tg + t * C + i0) = make_float4(tv[0], tv[1], tv[2], tv[3]);
            *reinterpret_cast<float4 *>(Tg + t * C + i0 + 4) = make_float4(tv[4], tv[5], tv[6], tv[7]);
            *reinterpret_cast<float4 *>(Pg + t * C + i0) = make_float4(pv[0], pv[1], pv[2], pv[3]);
            *reinterpret_cast<float4 *>(Pg + t * C + i0 + 4) = make_float4(pv[4], pv[5], pv[6], pv[7]);
        } else {
            uint16_t *Th = reinterpret_cast<uint16_t *>(wsu);
            uint4 hi, lo;
            split8(tv, hi, lo);
            *reinterpret_cast<uint4 *>(Th + t * C + i0) = hi;
            *reinterpret_cast<uint4 *>(Th + C * C + t * C + i0) = lo;
            split8(pv, hi, lo);
            *reinterpret_cast<uint4 *>(Th + 2 * C * C + t * C + i0) = hi;
            *reinterpret_cast<uint4 *>(Th + 3 * C * C + t * C + i0) = lo;
        }
    }
    if (tid < C) {
        gg[tid] = (float)gs[tid];
        gg[C + tid] = exp2_fast((float)gs[tid]);
        gg[2 * C + tid] = exp2_fast((float)(gs[C - 1] - gs[tid]));   // rows past the ragged end keep g constant
    }
}

// ---------------------------------------------------------------------------
// Scan, fp32 inputs (fp32 matrix cores): state carried across the chunks of
// one (b, h) unit for BV columns.  Workgroup layout: 4 waves; wave w owns output row tile I = w % (C/16) and the
// column tiles J of the output tiles o = w + 4m (o = I + (C/16) J); the state
// tiles s = w + 4m (s = (dk tile) * (BV/16) + J) share one column tile.
// ---------------------------------------------------------------------------
template <int DK, int C, int BV, int PREC, typename TI>
struct ScanPrefetch {
    static constexpr int NTR = C / 16;
    static constexpr int NT_O = NTR * (BV / 16);
    static constexpr int MAXO = (NT_O + 3) / 4;
    static constexpr int NKB_C = (C + 31) / 32;
    static constexpr int KL = (C * (DK / 8) + 255) / 256;
    Raw8<TI> k[KL];            // K rows for the LDS copy
    Raw8<TI> qf[DK / 32];      // Q fragments of the wave's row tile
    Frag tf[NKB_C], pf[NKB_C]; // Tm and P fragments of the wave's row tile
    TI v[MAXO][4];             // V entries of the wave's output tiles (raw)
    float e, w;                // 2^g[tid], 2^(gC - g[tid]) (tid < C)
};

template <int DK, int DV, int BV, int C, int PREC, typename TI, typename TO>
__global__ __launch_bounds__(256) void scan_head_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                        const TI *__restrict__ v, const float *__restrict__ ws,
                                                        const float *__restrict__ state_in, TO *__restrict__ out,
                                                        float *__restrict__ state_out, int L, int H, int NC) {
    using PF = ScanPrefetch<DK, C, BV, PREC, TI>;
    constexpr int KP = DK + 4;
    constexpr int CP = C + 4;
    constexpr int NTR = C / 16, NTV = BV / 16, NTK = DK / 16;
    constexpr int NT_O = NTR * NTV, NT_S = NTK * NTV;
    constexpr int MAXO = (NT_O + 3) / 4, MAXS = (NT_S + 3) / 4;
    constexpr int NKB_C = (C + 31) / 32;
    constexpr int NV = DV / BV;
    static_assert(4 % NTR == 0, "a wave's output tiles share one row tile");
    static_assert(4 % NTV == 0 && NT_S % 4 == 0, "a wave's state tiles share one column tile");

    __shared__ __attribute__((aligned(16))) float Ks[C * KP];
    __shared__ __attribute__((aligned(16))) float St[BV * KP];
    __shared__ __attribute__((aligned(16))) float Rt[BV * CP];
    __shared__ __attribute__((aligned(16))) float Ut[BV * CP];
    __shared__ __attribute__((aligned(16))) float U2t[BV * CP];
    __shared__ float es[C], ws2[C];   // 2^g and 2^(gC - g) of the current chunk

    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    const int vb = logical % NV;
    const size_t unit = logical / NV;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const int v0 = vb * BV;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const int I = wave % NTR;                       // this wave's output row tile
    const bool has_o = wave < NT_O;
    const int nkb = (16 * I + 16 + 31) / 32;        // K-blocks at or below the diagonal of row tile I
    const size_t tok_stride = (size_t)H;            // tokens are [B, L, H, d]
    const size_t base_tok = (size_t)b * L * tok_stride + h;

    // Every load below is unconditional and unmasked: row indices past the
    // ragged end are clamped to the last valid row, and the values are zeroed
    // where they are consumed (one chunk later).  A select or a branch next to
    // the load would make the wave wait for it here and defeat the prefetch.
    auto fetch = [&](int n, PF &p) {
        const int t0 = n * C;
        const int Lc = min(C, L - t0);
#pragma unroll
        for (int i = 0; i < PF::KL; ++i) {
            const int idx = min(tid + 256 * i, C * (DK / 8) - 1);
            const int t = idx / (DK / 8), c8 = idx % (DK / 8);
            load_raw8<TI>(p.k[i], k + (base_tok + (size_t)(t0 + min(t, Lc - 1)) * tok_stride) * DK + 8 * c8);
        }
        const int trow_c = min(16 * I + lr, Lc - 1);
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
            load_raw8<TI>(p.qf[kb], q + (base_tok + (size_t)(t0 + trow_c) * tok_stride) * DK + 32 * kb + 8 * lq);
        const float *wsu = ws + (unit * NC + n) * (size_t)(2 * C * C + 3 * C);
#pragma unroll
        for (int kb = 0; kb < NKB_C; ++kb) {
            const int kcc = min(32 * kb + 8 * lq, C - 8);
            load_frag_f32(p.tf[kb], wsu + (16 * I + lr) * C + kcc);
            load_frag_f32(p.pf[kb], wsu + C * C + (16 * I + lr) * C + kcc);
        }
#pragma unroll
        for (int m = 0; m < MAXO; ++m) {
            const int o = min(wave + 4 * m, NT_O - 1);
            const int J = o / NTR;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + 4 * lq + r;
                p.v[m][r] = v[(base_tok + (size_t)(t0 + min(t, Lc - 1)) * tok_stride) * DV + v0 + 16 * J + lr];
            }
        }
        p.e = wsu[2 * C * C + C + min(tid, C - 1)];
        p.w = wsu[2 * C * C + 2 * C + min(tid, C - 1)];
    };

    // initial state -> registers (state tiles) and St (transposed)
    f32x4 Sacc[MAXS];
#pragma unroll
    for (int m = 0; m < MAXS; ++m) {
        const int s = wave + 4 * m;
        Sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s < NT_S) {
            const int Ik = s / NTV, J = s % NTV;
            if (state_in) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Sacc[m][r] = state_in[(unit * DK + 16 * Ik + 4 * lq + r) * DV + v0 + 16 * J + lr];
            }
            *reinterpret_cast<float4 *>(St + (16 * J + lr) * KP + 16 * Ik + 4 * lq) =
                make_float4(Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
        }
    }

    // bf16: the next chunk's inputs are fetched while this chunk computes.
    // fp32 (not pipelined): each chunk fetches its own inputs first.
    constexpr bool PIPE = PREC == PREC_BF16;
    PF cur, nxt;
    if constexpr (PIPE) fetch(0, cur);
    for (int n = 0; n < NC; ++n) {
        const int t0 = n * C;
        const int Lc = min(C, L - t0);
        if constexpr (!PIPE) fetch(n, cur);
        __syncthreads();   // the previous chunk is done with Ks and gs; St is complete
#pragma unroll
        for (int i = 0; i < PF::KL; ++i) {
            const int idx = tid + 256 * i;
            if (idx < C * (DK / 8)) {
                const int t = idx / (DK / 8), c8 = idx % (DK / 8);
                Frag f;
                raw_to_frag(f, cur.k[i]);
                if (t >= Lc) zero_frag(f);
                float *pk = Ks + t * KP + 8 * c8;
                *reinterpret_cast<float4 *>(pk) = make_float4(f.x[0], f.x[1], f.x[2], f.x[3]);
                *reinterpret_cast<float4 *>(pk + 4) = make_float4(f.x[4], f.x[5], f.x[6], f.x[7]);
            }
        }
        if (tid < C) { es[tid] = cur.e; ws2[tid] = cur.w; }
        __syncthreads();
        if constexpr (PIPE) {
            if (n + 1 < NC) fetch(n + 1, nxt);   // in flight during this chunk
        }

        // X_K = K S, X_Q = Q S;  R = V - e^g X_K (to LDS);  O = e^g X_Q (registers)
        f32x4 xk[MAXO], xq[MAXO], Oacc[MAXO];
#pragma unroll
        for (int m = 0; m < MAXO; ++m) {
            xk[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            xq[m] = xk[m];
            Oacc[m] = xk[m];
        }
        if (has_o) {
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag fk, fq;
                load_frag_f32(fk, Ks + (16 * I + lr) * KP + 32 * kb + 8 * lq);
                raw_to_frag(fq, cur.qf[kb]);
                if (16 * I + lr >= Lc) zero_frag(fq);
                const auto ak = make_op<PREC, true>(fk);
                const auto aq = make_op<PREC, true>(fq);
#pragma unroll
                for (int m = 0; m < MAXO; ++m) {
                    const int o = wave + 4 * m;
                    if (o >= NT_O) continue;
                    const int J = o / NTR;
                    Frag fs;
                    load_frag_f32(fs, St + (16 * J + lr) * KP + 32 * kb + 8 * lq);
                    const auto bsop = make_op<PREC, false>(fs);
                    mma_op<PREC, true, false>(xk[m], ak, bsop);
                    mma_op<PREC, true, false>(xq[m], aq, bsop);
                }
            }
            float eg[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) eg[r] = es[16 * I + 4 * lq + r];
#pragma unroll
            for (int m = 0; m < MAXO; ++m) {
                const int o = wave + 4 * m;
                if (o >= NT_O) continue;
                const int J = o / NTR;
                float rr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float vv = (16 * I + 4 * lq + r < Lc) ? to_f32(cur.v[m][r]) : 0.f;
                    rr[r] = vv - eg[r] * xk[m][r];
                    Oacc[m][r] = eg[r] * xq[m][r];
                }
                *reinterpret_cast<float4 *>(Rt + (16 * J + lr) * CP + 16 * I + 4 * lq) =
                    make_float4(rr[0], rr[1], rr[2], rr[3]);
            }
        }
        __syncthreads();

        // U = Tm R;  Ut = U, U2t = e^{g_C - g} U
        if (has_o) {
            f32x4 ua[MAXO];
#pragma unroll
            for (int m = 0; m < MAXO; ++m) ua[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB_C; ++kb) {
                if (kb >= nkb) continue;
                const int kc = 32 * kb + 8 * lq;
                Frag ft = cur.tf[kb];
                if (kc >= C) zero_frag(ft);
                const auto at = make_op<PREC, false>(ft);
#pragma unroll
                for (int m = 0; m < MAXO; ++m) {
                    const int o = wave + 4 * m;
                    if (o >= NT_O) continue;
                    const int J = o / NTR;
                    Frag fb;
                    load_frag_f32(fb, Rt + (16 * J + lr) * CP + min(kc, C - 8));
                    if (kc >= C) zero_frag(fb);
                    mma_op<PREC, false, false>(ua[m], at, make_op<PREC, false>(fb));
                }
            }
            float w2[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) w2[r] = ws2[16 * I + 4 * lq + r];
#pragma unroll
            for (int m = 0; m < MAXO; ++m) {
                const int o = wave + 4 * m;
                if (o >= NT_O) continue;
                const int J = o / NTR;
                *reinterpret_cast<float4 *>(Ut + (16 * J + lr) * CP + 16 * I + 4 * lq) =
                    make_float4(ua[m][0], ua[m][1], ua[m][2], ua[m][3]);
                *reinterpret_cast<float4 *>(U2t + (16 * J + lr) * CP + 16 * I + 4 * lq) =
                    make_float4(w2[0] * ua[m][0], w2[1] * ua[m][1], w2[2] * ua[m][2], w2[3] * ua[m][3]);
            }
        }
        __syncthreads();

        // O += P U, store
        if (has_o) {
#pragma unroll
            for (int kb = 0; kb < NKB_C; ++kb) {
                if (kb >= nkb) continue;
                const int kc = 32 * kb + 8 * lq;
                Frag fp = cur.pf[kb];
                if (kc >= C) zero_frag(fp);
                const auto ap = make_op<PREC, false>(fp);
#pragma unroll
                for (int m = 0; m < MAXO; ++m) {
                    const int o = wave + 4 * m;
                    if (o >= NT_O) continue;
                    const int J = o / NTR;
                    Frag fb;
                    load_frag_f32(fb, Ut + (16 * J + lr) * CP + min(kc, C - 8));
                    if (kc >= C) zero_frag(fb);
                    mma_op<PREC, false, false>(Oacc[m], ap, make_op<PREC, false>(fb));
                }
            }
#pragma unroll
            for (int m = 0; m < MAXO; ++m) {
                const int o = wave + 4 * m;
                if (o >= NT_O) continue;
                const int J = o / NTR;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * I + 4 * lq + r;
                    if (t < Lc) store1<TO>(out + (base_tok + (size_t)(t0 + t) * tok_stride) * DV + v0 + 16 * J + lr, Oacc[m][r]);
                }
            }
        }

        // S <- e^{g_C} S + K^T U2   (the wave's state tiles share column tile J = wave % NTV)
        const float eC = es[Lc - 1];
        const int Js = wave % NTV;
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[m][r] *= eC;
        }
#pragma unroll
        for (int kb = 0; kb < NKB_C; ++kb) {
            const int kc = 32 * kb + 8 * lq;
            Frag fb;
            load_frag_f32(fb, U2t + (16 * Js + lr) * CP + min(kc, C - 8));
            if (kc >= C) zero_frag(fb);
            const auto bu = make_op<PREC, false>(fb);
#pragma unroll
            for (int m = 0; m < MAXS; ++m) {
                const int s = wave + 4 * m;
                const int Ik = s / NTV;
                Frag fa;
                load_frag_strided(fa, Ks + min(kc, C - 8) * KP + 16 * Ik + lr, KP);
                if (kc >= C) zero_frag(fa);
                mma_op<PREC, true, false>(Sacc[m], make_op<PREC, true>(fa), bu);
            }
        }
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
            const int s = wave + 4 * m;
            const int Ik = s / NTV;
            *reinterpret_cast<float4 *>(St + (16 * Js + lr) * KP + 16 * Ik + 4 * lq) =
                make_float4(Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
        }
        if constexpr (PIPE) {
            if (n + 1 < NC) cur = nxt;
        }
    }

    if (state_out) {
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
            const int s = wave + 4 * m;
            const int Ik = s / NTV, J = s % NTV;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                state_out[(unit * DK + 16 * Ik + 4 * lq + r) * DV + v0 + 16 * J + lr] = Sacc[m][r];
        }
    }
}


// ---------------------------------------------------------------------------
// Scan, bf16 inputs: 8 waves (two per SIMD) per (b, h, BV-column block).
//  * Every matrix-core operand is read from LDS as bf16: K, Q raw, and the fp32
//    intermediates S^T, R^T, U^T, U2^T as hi/lo pairs written by the one wave
//    that produces them.  K^T fragments for the state update come straight
//    from the row-major K tile through LDS transpose reads (ds_read_b64_tr_b16):
//    within each 16-lane group, lane 4e+m points at K[t0 + e][c0 + 4m] and lane
//    4m+s receives K[t0 + 0..3][c0 + 4m + s].
//  * fp32 x fp32 products take hi*hi + lo*hi + hi*lo; q, k are bf16-exact.
//  * Staging: the next chunk's K, Q, V columns, Tm, P (hi/lo) and decay vectors
//    are fetched while the current chunk computes, with coalesced 16-byte loads
//    that fetch every byte once per block, and parked in registers.  K, Q, V and
//    the decay vectors go to LDS at the end of the chunk (K double-buffered, as
//    the state update still reads the current tile), Tm and P after the next
//    chunk's first barrier, when the current ones have been read.
//  * The output tile is staged in LDS and written with 16-byte stores after the
//    next chunk's first barrier, behind that chunk's loads: vector-memory
//    counters retire in issue order, so a store would otherwise hold up the
//    wait for every load issued after it.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((address_space(3))) short4_t lds_short4;

// 16 bytes of staged outputs times their gate values: 8 bf16 outputs times 8
// bf16 gates, or 4 fp32 outputs times the 4 bf16 gates in the first 8 bytes.
template <typename TO>
__device__ __forceinline__ u32x4 gate_outputs(u32x4 x, u32x4 g);
template <>
__device__ __forceinline__ u32x4 gate_outputs<uint16_t>(u32x4 x, u32x4 g) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(x[i] << 16) * __uint_as_float(g[i] << 16);
        const float hi = __uint_as_float(x[i] & 0xFFFF0000u) * __uint_as_float(g[i] & 0xFFFF0000u);
        r[i] = (uint32_t)bf16_bits(lo) | ((uint32_t)bf16_bits(hi) << 16);
    }
    return r;
}
template <>
__device__ __forceinline__ u32x4 gate_outputs<float>(u32x4 x, u32x4 g) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t gw = g[i / 2];
        const float gv = __uint_as_float((i & 1) ? (gw & 0xFFFF0000u) : (gw << 16));
        r[i] = __float_as_uint(__uint_as_float(x[i]) * gv);
    }
    return r;
}

template <int DK, int DV, int BV, int C, typename TO>
__global__ __launch_bounds__(512) void scan_head_bf16_kernel(const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ k,
                                                             const uint16_t *__restrict__ v,
                                                             const unsigned char *__restrict__ ws,
                                                             const float *__restrict__ state_in,
                                                             TO *__restrict__ out, float *__restrict__ state_out,
                                                             int L, int H, int NC,
                                                             const uint16_t *__restrict__ gate) {
    constexpr int NW = 8, NTH = 64 * NW;
    // bf16 pitch of K, Q and S^T rows: DK + 8 puts consecutive rows 4 banks apart,
    // so a 16-row fragment read (16 bytes per row) touches 64 distinct banks; it
    // costs the 4-row transpose reads of K a 2-way overlap, which measured cheaper
    // (scan 197 vs 210 us on the headline workload with rows 8 banks apart)
    constexpr int KP = DK + 8;
    constexpr int CP = C + 16;   // bf16 pitch of Tm, P, R^T, U^T, U2^T rows (measured best of C + 8/16/24)
    constexpr int VP = BV + 8;   // bf16 pitch of V rows
    constexpr int OV = 16 / (int)sizeof(TO);   // outputs per 16-byte store
    constexpr int OP = BV + OV;                // pitch of the staged output rows
    constexpr int NTR = C / 16, NTV = BV / 16, NTK = DK / 16;
    constexpr int NT_O = NTR * NTV, NT_S = NTK * NTV;
    constexpr int MAXS = NT_S / NW;
    constexpr int NKB_C = (C + 31) / 32;
    constexpr int NV = DV / BV;
    constexpr int WSB = 8 * C * C + 12 * C;    // workspace bytes per chunk
    // 16-byte pieces per chunk: K (and Q), V columns, Tm/P hi/lo, decay vectors, outputs
    constexpr int NK = C * DK / 8, KL = (NK + NTH - 1) / NTH;
    constexpr int NVP = C * BV / 8;
    constexpr int NF = C * C / 2, FL = (NF + NTH - 1) / NTH;
    constexpr int NG = C / 2;
    constexpr int NO = C * BV / OV;
    static_assert(NT_O <= NW && NT_S % NW == 0 && NW % NTV == 0, "scan tiling");
    static_assert(KL <= 2 && FL <= 4 && NVP <= NTH && NO <= NTH && NG <= 64, "staging");
    static_assert(NK % 64 == 0 && NVP % 64 == 0 && NF % 64 == 0 && NO % 64 == 0, "whole waves per piece set");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Qs[C * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[C * VP];
    __shared__ __attribute__((aligned(16))) uint16_t Fs[4 * C * CP];   // Tm hi, Tm lo, P hi, P lo
    __shared__ __attribute__((aligned(16))) float Gs[2 * C];           // 2^g, 2^(gC - g)
    __shared__ __attribute__((aligned(16))) uint16_t Sth[BV * KP], Stl[BV * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Rth[BV * CP], Rtl[BV * CP];
    __shared__ __attribute__((aligned(16))) uint16_t Uth[BV * CP], Utl[BV * CP];
    __shared__ __attribute__((aligned(16))) uint16_t U2h[BV * CP], U2l[BV * CP];
    __shared__ __attribute__((aligned(16))) TO Os[C * OP];

    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    const int vb = logical % NV;
    const size_t unit = logical / NV;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const int v0 = vb * BV;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    const bool has_o = NT_O == NW || wave < NT_O;
    const int ot = has_o ? wave : NT_O - 1;
    const int I = ot % NTR, J = ot / NTR;          // this wave's output tile
    const int Js = wave % NTV;                     // column tile of this wave's state tiles
    const unsigned tok_stride = (unsigned)H * DK;  // elements between consecutive tokens (q, k)
    const unsigned vtok_stride = (unsigned)H * DV;
    const uint16_t *kb_ptr = k + ((size_t)b * L * H + h) * DK;   // token 0 of this unit
    const uint16_t *qb_ptr = q + ((size_t)b * L * H + h) * DK;
    const uint16_t *vb_ptr = v + ((size_t)b * L * H + h) * DV + v0;
    TO *ob_ptr = out + ((size_t)b * L * H + h) * DV + v0;
    const uint16_t *gb_ptr = gate ? gate + ((size_t)b * L * H + h) * DV + v0 : nullptr;
    // transpose-read lane roles: e = token offset, m = channel quad (see above)
    const int tr_e = (lane & 15) >> 2, tr_m = lane & 3, tr_g = lane >> 4;

    // Staging roles of this thread (fixed for the whole scan).
    int krow[KL], kcol[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) {
        const int idx = min(tid + NTH * i, NK - 1);
        krow[i] = idx / (DK / 8);
        kcol[i] = 8 * (idx % (DK / 8));
    }
    const int vidx = min(tid, NVP - 1);
    const int vrow = vidx / (BV / 8), vcol = 8 * (vidx % (BV / 8));
    int fl[FL];   // LDS offsets of this thread's Tm/P pieces
#pragma unroll
    for (int i = 0; i < FL; ++i) {
        const int idx = min(tid + NTH * i, NF - 1);
        const int arr = idx / (C * C / 8), rem = idx % (C * C / 8);
        fl[i] = arr * C * CP + (rem / (C / 8)) * CP + 8 * (rem % (C / 8));
    }
    const int gidx = min(lane, NG - 1);
    const int orow = min(tid, NO - 1) / (BV / OV), ocol = OV * (min(tid, NO - 1) % (BV / OV));

    u32x4 rk[KL], rq[KL], rv, rf[FL], rg, rgate = {0u, 0u, 0u, 0u};
    // Loads of chunk n's inputs into the staging registers.  Rows past the end
    // of a ragged last chunk repeat its last token: beta is zero there, so Tm
    // has zero rows and columns for them and they never reach an output.
    // With an output gate, the gate values of chunk gn's outputs come first:
    // they are stored at the top of chunk gn + 1, and by then every load of this
    // fetch has been waited for (so the store waits for none of the later ones).
    auto fetch = [&](int n, int gn) __attribute__((always_inline)) {
        if (gb_ptr && gn >= 0 && (NO == NTH || wave < NO / 64) && orow < min(C, L - gn * C)) {
            const uint16_t *gp = gb_ptr + ((size_t)gn * C + orow) * vtok_stride + ocol;   // OV gate values
            if constexpr (OV == 8) {
                rgate = *reinterpret_cast<const u32x4 *>(gp);
            } else {
                const uint2 g2 = *reinterpret_cast<const uint2 *>(gp);
                rgate[0] = g2.x;
                rgate[1] = g2.y;
            }
        }
        const int t0 = n * C;
        const int last = min(C, L - t0) - 1;
        const uint16_t *kc = kb_ptr + (size_t)t0 * tok_stride;
        const uint16_t *qc = qb_ptr + (size_t)t0 * tok_stride;
        const uint16_t *vc = vb_ptr + (size_t)t0 * vtok_stride;
        const unsigned char *wsu = ws + (unit * NC + (unsigned)n) * (size_t)WSB;
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            if (NTH * (i + 1) <= NK || wave < (NK - NTH * i) / 64) {
                const unsigned off = (unsigned)min(krow[i], last) * tok_stride + (unsigned)kcol[i];
                rk[i] = *reinterpret_cast<const u32x4 *>(kc + off);
                rq[i] = *reinterpret_cast<const u32x4 *>(qc + off);
            }
        }
        if (NVP == NTH || wave < NVP / 64)
            rv = *reinterpret_cast<const u32x4 *>(vc + (unsigned)min(vrow, last) * vtok_stride + (unsigned)vcol);
        if (wave == 0)
            rg = *reinterpret_cast<const u32x4 *>(wsu + 8 * C * C + 4 * C + 16 * gidx);   // [2^g | 2^(gC-g)]
#pragma unroll
        for (int i = 0; i < FL; ++i) {
            if (NTH * (i + 1) <= NF || wave < (NF - NTH * i) / 64)
                rf[i] = *reinterpret_cast<const u32x4 *>(wsu + 16 * (unsigned)(tid + NTH * i));
        }
    };
    auto stage_kqvg = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            if (NTH * (i + 1) <= NK || wave < (NK - NTH * i) / 64) {
                *reinterpret_cast<u32x4 *>(&Ks[buf][krow[i] * KP + kcol[i]]) = rk[i];
                *reinterpret_cast<u32x4 *>(&Qs[krow[i] * KP + kcol[i]]) = rq[i];
            }
        }
        if (NVP == NTH || wave < NVP / 64) *reinterpret_cast<u32x4 *>(&Vs[vrow * VP + vcol]) = rv;
        if (wave == 0) *reinterpret_cast<u32x4 *>(&Gs[4 * gidx]) = rg;
    };
    auto stage_f = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FL; ++i) {
            if (NTH * (i + 1) <= NF || wave < (NF - NTH * i) / 64)
                *reinterpret_cast<u32x4 *>(&Fs[fl[i]]) = rf[i];
        }
    };
    auto store_o = [&](int n, int rows) __attribute__((always_inline)) {   // staged outputs of chunk n
        if ((NO == NTH || wave < NO / 64) && orow < rows) {
            const unsigned off = (unsigned)orow * vtok_stride + (unsigned)ocol;
            TO *oc = ob_ptr + (size_t)n * C * vtok_stride;
            u32x4 x = *reinterpret_cast<const u32x4 *>(&Os[orow * OP + ocol]);
            // output gate of the looped block: o * sigmoid(z_g), bf16 gate values of chunk n
            if (gb_ptr) x = gate_outputs<TO>(x, rgate);
            *reinterpret_cast<u32x4 *>(oc + off) = x;
        }
    };
    auto store_split = [&](uint16_t *hi, uint16_t *lo, int off, const float x[4]) __attribute__((always_inline)) {
        uint2 h2, l2;
        split4(x, h2, l2);
        *reinterpret_cast<uint2 *>(hi + off) = h2;
        *reinterpret_cast<uint2 *>(lo + off) = l2;
    };

    // initial state: registers (state tiles) and S^T (hi/lo) in LDS
    f32x4 Sacc[MAXS];
#pragma unroll
    for (int m = 0; m < MAXS; ++m) {
        const int Ik = (wave + NW * m) / NTV;
        Sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (state_in) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sacc[m][r] = state_in[(unit * DK + 16 * Ik + 4 * lq + r) * DV + v0 + 16 * Js + lr];
        }
        const float x[4] = {Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]};
        store_split(Sth, Stl, (16 * Js + lr) * KP + 16 * Ik + 4 * lq, x);
    }
    fetch(0, -1);
    stage_kqvg(0);

    for (int n = 0; n < NC; ++n) {
        const int buf = n & 1;
        __syncthreads();   // chunk n's K, Q, V, decay vectors and S^T are in LDS; Tm, P and outputs of n - 1 are read
        stage_f();                     // Tm, P of chunk n (first read after the next barrier)
        if (n > 0) store_o(n - 1, C);  // only the last chunk can be ragged; gate values of n - 1 in rgate
        fetch(min(n + 1, NC - 1), n);  // the last chunk re-fetches itself (unused); gate values of chunk n

        // X_K = K S, X_Q = Q S;  R = V - 2^g X_K (hi/lo to LDS);  O = 2^g X_Q
        f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
        if (has_o) {
            f32x4 xk = {0.f, 0.f, 0.f, 0.f}, xq = xk;
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                const int ao = (16 * I + lr) * KP + 32 * kb + 8 * lq;
                const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(&Ks[buf][ao]);
                const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(&Qs[ao]);
                const int so = (16 * J + lr) * KP + 32 * kb + 8 * lq;
                const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(Sth + so);
                const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(Stl + so);
                xk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bh, xk, 0, 0, 0);
                xq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bh, xq, 0, 0, 0);
                xk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bl, xk, 0, 0, 0);
                xq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bl, xq, 0, 0, 0);
            }
            const f32x4 eg = *reinterpret_cast<const f32x4 *>(&Gs[16 * I + 4 * lq]);
            float rr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                rr[r] = bf16_to_f32(Vs[(16 * I + 4 * lq + r) * VP + 16 * J + lr]) - eg[r] * xk[r];
                oacc[r] = eg[r] * xq[r];
            }
            store_split(Rth, Rtl, (16 * J + lr) * CP + 16 * I + 4 * lq, rr);
        }
        __syncthreads();

        // U = Tm R;  U^T and U2^T = (2^(gC - g) U)^T as hi/lo
        const float ec = Gs[C - 1];   // 2^gC, read before the decay vectors are restaged
        if (has_o) {
            f32x4 ua = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB_C; ++kb) {   // blocks above the diagonal hold zeros
                const int kc = 32 * kb + 8 * lq;
                const bool kin = (C >= 32) || kc < C;
                const bf16x8 z = {};
                const int fo = (16 * I + lr) * CP + min(kc, C - 8);
                const bf16x8 th = kin ? *reinterpret_cast<const bf16x8 *>(&Fs[fo]) : z;
                const bf16x8 tl = kin ? *reinterpret_cast<const bf16x8 *>(&Fs[C * CP + fo]) : z;
                const int ro = (16 * J + lr) * CP + min(kc, C - 8);
                const bf16x8 rh = *reinterpret_cast<const bf16x8 *>(Rth + ro);
                const bf16x8 rl = *reinterpret_cast<const bf16x8 *>(Rtl + ro);
                ua = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th, rh, ua, 0, 0, 0);
                ua = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl, rh, ua, 0, 0, 0);
                ua = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th, rl, ua, 0, 0, 0);
            }
            const f32x4 ew = *reinterpret_cast<const f32x4 *>(&Gs[C + 16 * I + 4 * lq]);
            float u[4], w2[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                u[r] = ua[r];
                w2[r] = ew[r] * ua[r];
            }
            const int uo = (16 * J + lr) * CP + 16 * I + 4 * lq;
            store_split(Uth, Utl, uo, u);
            store_split(U2h, U2l, uo, w2);
        }
        __syncthreads();

        // O += P U, staged in LDS
        if (has_o) {
#pragma unroll
            for (int kb = 0; kb < NKB_C; ++kb) {
                const int kc = 32 * kb + 8 * lq;
                const bool kin = (C >= 32) || kc < C;
                const bf16x8 z = {};
                const int fo = (16 * I + lr) * CP + min(kc, C - 8);
                const bf16x8 ph = kin ? *reinterpret_cast<const bf16x8 *>(&Fs[2 * C * CP + fo]) : z;
                const bf16x8 pl = kin ? *reinterpret_cast<const bf16x8 *>(&Fs[3 * C * CP + fo]) : z;
                const int uo = (16 * J + lr) * CP + min(kc, C - 8);
                const bf16x8 uh = *reinterpret_cast<const bf16x8 *>(Uth + uo);
                const bf16x8 ul = *reinterpret_cast<const bf16x8 *>(Utl + uo);
                oacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, uh, oacc, 0, 0, 0);
                oacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, uh, oacc, 0, 0, 0);
                oacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, ul, oacc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) store1<TO>(&Os[(16 * I + 4 * lq + r) * OP + 16 * J + lr], oacc[r]);
        }

        // S <- 2^gC S + K^T U2  (K^T fragments by transpose reads of K[buf])
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[m][r] *= ec;
        }
#pragma unroll
        for (int kb = 0; kb < NKB_C; ++kb) {
            const int kc = 32 * kb + 8 * lq;
            const bool kin = (C >= 32) || kc < C;
            const int kcc = min(kc, C - 8);
            const bf16x8 z = {};
            const bf16x8 bh = kin ? *reinterpret_cast<const bf16x8 *>(U2h + (16 * Js + lr) * CP + kcc) : z;
            const bf16x8 bl = kin ? *reinterpret_cast<const bf16x8 *>(U2l + (16 * Js + lr) * CP + kcc) : z;
            // tokens of this lane group's fragment: 32 kb + 8 g .. + 7 (clamped for C = 16)
            const int tt = min(32 * kb + 8 * tr_g, C - 8);
#pragma unroll
            for (int m = 0; m < MAXS; ++m) {
                const int Ik = (wave + NW * m) / NTV;
                const int col = 16 * Ik + 4 * tr_m;
                const short4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4 *)(&Ks[buf][(tt + tr_e) * KP + col]));
                const short4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4 *)(&Ks[buf][(tt + 4 + tr_e) * KP + col]));
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, (__attribute__((ext_vector_type(8))) short){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1],
                                                                        hi4[2], hi4[3]});
                Sacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, Sacc[m], 0, 0, 0);
                Sacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, Sacc[m], 0, 0, 0);
            }
        }
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
            const int Ik = (wave + NW * m) / NTV;
            const float x[4] = {Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]};
            store_split(Sth, Stl, (16 * Js + lr) * KP + 16 * Ik + 4 * lq, x);
        }
        stage_kqvg(buf ^ 1);   // chunk n + 1's inputs; their current copies were last read before the second barrier
    }
    __syncthreads();
    store_o(NC - 1, L - (NC - 1) * C);

    if (state_out) {
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
            const int Ik = (wave + NW * m) / NTV;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                state_out[(unit * DK + 16 * Ik + 4 * lq + r) * DV + v0 + 16 * Js + lr] = Sacc[m][r];
        }
    }
}

size_t prefill_head_ws_bytes(int B, int L, int H, int C) {
    const size_t NC = (size_t)((L + C - 1) / C);
    return (size_t)B * H * NC * (size_t)(8 * C * C + 12 * C);
}

template <int D, int C, int PREC, typename TI, typename TO>
static hipError_t run(const GdnArgs &a, int phase, hipStream_t s) {
    constexpr int BV = 32;
    const int NC = (a.L + C - 1) / C;
    const unsigned units = (unsigned)a.B * (unsigned)a.H;
    if (phase & PHASE_PREPARE) {
        hipLaunchKernelGGL((prep_head_kernel<D, C, PREC, TI>), dim3(units * NC), dim3(256), 0, s,
                           (const TI *)a.q, (const TI *)a.k, a.alpha, a.beta, (unsigned char *)a.ws, a.L, a.H, NC);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & PHASE_SCAN) {
        if constexpr (PREC == PREC_BF16) {
            // 32-column blocks, or (d = 128, C = 64) 16-column blocks when 32
            // would leave compute units idle: each block walks every chunk of its
            // unit and loads the chunk's K, Q, Tm and P either way, but twice the
            // blocks run at once
            if constexpr (D == 128 && C == 64) {
                if ((long)units * (D / BV) < device_cus()) {
                    hipLaunchKernelGGL((scan_head_bf16_kernel<D, D, BV / 2, C, TO>), dim3(units * (D / (BV / 2))),
                                       dim3(512), 0, s, (const uint16_t *)a.q, (const uint16_t *)a.k,
                                       (const uint16_t *)a.v, (const unsigned char *)a.ws, a.state_in, (TO *)a.out,
                                       a.state_out, a.L, a.H, NC, a.gate);
                    return hipGetLastError();
                }
            }
            hipLaunchKernelGGL((scan_head_bf16_kernel<D, D, BV, C, TO>), dim3(units * (D / BV)), dim3(512), 0, s,
                               (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                               (const unsigned char *)a.ws, a.state_in, (TO *)a.out, a.state_out, a.L, a.H, NC,
                               a.gate);
        } else {
            hipLaunchKernelGGL((scan_head_kernel<D, D, BV, C, PREC, TI, TO>), dim3(units * (D / BV)), dim3(256), 0, s,
                               (const TI *)a.q, (const TI *)a.k, (const TI *)a.v, (const float *)a.ws, a.state_in,
                               (TO *)a.out, a.state_out, a.L, a.H, NC);
        }
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int D, int C>
static hipError_t run_t(const GdnArgs &a, int phase, hipStream_t s) {
    if (a.qkv_bf16)
        return a.out_bf16 ? run<D, C, PREC_BF16, uint16_t, uint16_t>(a, phase, s)
                          : run<D, C, PREC_BF16, uint16_t, float>(a, phase, s);
    return a.out_bf16 ? run<D, C, PREC_F32, float, uint16_t>(a, phase, s) : run<D, C, PREC_F32, float, float>(a, phase, s);
}

template <int D>
static hipError_t run_c(const GdnArgs &a, int phase, hipStream_t s) {
    switch (a.chunk) {
        case 16: return run_t<D, 16>(a, phase, s);
        case 32: return run_t<D, 32>(a, phase, s);
        default: return run_t<D, 64>(a, phase, s);
    }
}

hipError_t launch_prefill_head(const GdnArgs &a, int phase, hipStream_t s) {
    return a.dk == 64 ? run_c<64>(a, phase, s) : run_c<128>(a, phase, s);
}

}  // namespace lt2
