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
// Tm and P do not depend on the state: kernel 1 forms them for every chunk in
// parallel; kernel 2 carries the fp32 state across the chunks of one unit in
// order, for one block of BV state columns (columns evolve independently).
//
// Gate exponents are masked before exp, so every exponent is <= 0.
#include "common.h"
#include "internal.h"

namespace lt2 {

// ---------------------------------------------------------------------------
// Kernel 1: per chunk, Tm = (I + A)^{-1} diag(beta), P, and g.  Workspace per
// (b, h, chunk): Tm [C][C], P [C][C], g [C], fp32, zero above the diagonal.
// ---------------------------------------------------------------------------
template <int DK, int C, int PREC, typename TI>
__global__ __launch_bounds__(256) void prep_head_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                        const float *__restrict__ alpha,
                                                        const float *__restrict__ beta, float *__restrict__ ws,
                                                        int L, int H, int NC) {
    constexpr int KP = DK + 4;
    constexpr int CP = C + 4;
    constexpr int NT = C / 16;
    __shared__ __attribute__((aligned(16))) float Ks[C * KP];
    __shared__ __attribute__((aligned(16))) float Qs[C * KP];
    __shared__ float Am[C * CP];
    __shared__ float Ti[C * CP];
    __shared__ float Xs[4][16 * 17];
    __shared__ float gs[C], bs[C];

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = n * C;
    const int Lc = min(C, L - t0);
    float *wsu = ws + (((size_t)b * H + h) * NC + n) * (size_t)(2 * C * C + C);
    float *Tg = wsu, *Pg = wsu + C * C, *gg = wsu + 2 * C * C;

    for (int idx = tid; idx < C * (DK / 8); idx += 256) {
        const int t = idx / (DK / 8), c8 = idx % (DK / 8);
        Frag fk, fq;
        if (t < Lc) {
            const size_t off = ((size_t)(b * (size_t)L + t0 + t) * H + h) * DK + 8 * c8;
            load_row8<TI>(fk, k + off);
            load_row8<TI>(fq, q + off);
        } else {
            zero_frag(fk);
            zero_frag(fq);
        }
        float *pk = Ks + t * KP + 8 * c8, *pq = Qs + t * KP + 8 * c8;
        *reinterpret_cast<float4 *>(pk) = make_float4(fk.x[0], fk.x[1], fk.x[2], fk.x[3]);
        *reinterpret_cast<float4 *>(pk + 4) = make_float4(fk.x[4], fk.x[5], fk.x[6], fk.x[7]);
        *reinterpret_cast<float4 *>(pq) = make_float4(fq.x[0], fq.x[1], fq.x[2], fq.x[3]);
        *reinterpret_cast<float4 *>(pq + 4) = make_float4(fq.x[4], fq.x[5], fq.x[6], fq.x[7]);
    }
    if (wave == 0) {
        float lg = 0.f, bt = 0.f;
        if (lane < Lc) {
            const size_t tok = (size_t)(b * (size_t)L + t0 + lane) * H + h;
            lg = log_gate(alpha[tok]);
            bt = beta[tok];
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(lg, off);
            if (lane >= off) lg += y;
        }
        if (lane < C) { gs[lane] = lg; bs[lane] = bt; }
    }
    __syncthreads();

    // Gated K K^T (strictly lower, rows scaled by beta) into Am; gated Q K^T
    // (lower incl.) straight to the workspace.  Upper tiles are zero.
    for (int tt = wave; tt < 2 * NT * NT; tt += 4) {
        const int which = tt / (NT * NT);  // 0: KK^T, 1: QK^T
        const int I = (tt % (NT * NT)) / NT, J = tt % NT;
        const int row = 4 * (lane >> 4), col = lane & 15;
        if (J > I) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (which == 0) Am[(16 * I + row + r) * CP + 16 * J + col] = 0.f;
                else Pg[(16 * I + row + r) * C + 16 * J + col] = 0.f;
            }
            continue;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const float *Asrc = which == 0 ? Ks : Qs;
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            Frag fa, fb;
            load_frag_f32(fa, Asrc + (16 * I + (lane & 15)) * KP + 32 * kb + 8 * (lane >> 4));
            load_frag_f32(fb, Ks + (16 * J + (lane & 15)) * KP + 32 * kb + 8 * (lane >> 4));
            mma<PREC, true, true>(acc, fa, fb);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + row + r, i = 16 * J + col;
            if (which == 0) {
                Am[t * CP + i] = (i < t) ? bs[t] * expf(gs[t] - gs[i]) * acc[r] : 0.f;
            } else {
                Pg[t * C + i] = (i <= t && t < Lc) ? expf(gs[t] - gs[i]) * acc[r] : 0.f;
            }
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
            const int lr = lane & 15, lk = lane >> 4;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int Kb = J; Kb < I; ++Kb) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float a = Am[(16 * I + lr) * CP + 16 * Kb + 4 * kk + lk];
                    const float bb = Ti[(16 * Kb + 4 * kk + lk) * CP + 16 * J + lr];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Xs[wave][(4 * lk + r) * 17 + lr] = acc[r];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float a = Ti[(16 * I + lr) * CP + 16 * I + 4 * kk + lk];
                const float bb = Xs[wave][(4 * kk + lk) * 17 + lr];
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, y, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Ti[(16 * I + 4 * lk + r) * CP + 16 * J + lr] = -y[r];
        }
        __syncthreads();
    }

    // Tm = T diag(beta), zero above the diagonal.
    for (int idx = tid; idx < C * C; idx += 256) {
        const int t = idx / C, i = idx % C;
        Tg[idx] = (i <= t) ? Ti[t * CP + i] * bs[i] : 0.f;
    }
    if (tid < C) gg[tid] = gs[tid];
}

// ---------------------------------------------------------------------------
// Kernel 2: state scan over the chunks of one (b, h) unit for BV columns.
// ---------------------------------------------------------------------------
template <int DK, int DV, int BV, int C, int PREC, typename TI, typename TO>
__global__ __launch_bounds__(256) void scan_head_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                        const TI *__restrict__ v, const float *__restrict__ ws,
                                                        const float *__restrict__ state_in, TO *__restrict__ out,
                                                        float *__restrict__ state_out, int L, int H, int NC) {
    constexpr int KP = DK + 4;
    constexpr int CP = C + 4;
    constexpr int NTR = C / 16, NTV = BV / 16, NTK = DK / 16;
    constexpr int NT_O = NTR * NTV, NT_S = NTK * NTV;
    constexpr int MAXO = (NT_O + 3) / 4, MAXS = (NT_S + 3) / 4;
    constexpr int NKB_C = (C + 31) / 32;

    __shared__ __attribute__((aligned(16))) float Ks[C * KP];
    __shared__ __attribute__((aligned(16))) float St[BV * KP];
    __shared__ __attribute__((aligned(16))) float Rt[BV * CP];
    __shared__ __attribute__((aligned(16))) float Ut[BV * CP];
    __shared__ __attribute__((aligned(16))) float U2t[BV * CP];
    __shared__ float gs[C];

    const int vb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int v0 = vb * BV;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const size_t unit = (size_t)b * H + h;

    f32x4 Sacc[MAXS];
#pragma unroll
    for (int m = 0; m < MAXS; ++m) {
        const int s = wave + 4 * m;
        Sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s < NT_S && state_in) {
            const int Ik = s / NTV, J = s % NTV;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sacc[m][r] = state_in[(unit * DK + 16 * Ik + 4 * lq + r) * DV + v0 + 16 * J + lr];
        }
        if (s < NT_S) {
            const int Ik = s / NTV, J = s % NTV;
            *reinterpret_cast<float4 *>(St + (16 * J + lr) * KP + 16 * Ik + 4 * lq) =
                make_float4(Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
        }
    }

    for (int n = 0; n < NC; ++n) {
        const int t0 = n * C;
        const int Lc = min(C, L - t0);
        const float *wsu = ws + (unit * NC + n) * (size_t)(2 * C * C + C);
        const float *Tg = wsu, *Pg = wsu + C * C, *gg = wsu + 2 * C * C;
        __syncthreads();
        for (int idx = tid; idx < C * (DK / 8); idx += 256) {
            const int t = idx / (DK / 8), c8 = idx % (DK / 8);
            Frag fk;
            if (t < Lc) load_row8<TI>(fk, k + ((size_t)(b * (size_t)L + t0 + t) * H + h) * DK + 8 * c8);
            else zero_frag(fk);
            float *pk = Ks + t * KP + 8 * c8;
            *reinterpret_cast<float4 *>(pk) = make_float4(fk.x[0], fk.x[1], fk.x[2], fk.x[3]);
            *reinterpret_cast<float4 *>(pk + 4) = make_float4(fk.x[4], fk.x[5], fk.x[6], fk.x[7]);
        }
        if (tid < C) gs[tid] = gg[tid];
        __syncthreads();

        // X_K = K S, X_Q = Q S;  R = V - e^g X_K (to LDS);  O = e^g X_Q (registers)
        f32x4 Oacc[MAXO];
#pragma unroll
        for (int m = 0; m < MAXO; ++m) {
            const int o = wave + 4 * m;
            Oacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (o >= NT_O) continue;
            const int I = o / NTV, J = o % NTV;
            f32x4 xk = {0.f, 0.f, 0.f, 0.f}, xq = {0.f, 0.f, 0.f, 0.f};
            const int trow = 16 * I + lr;
            const TI *qrow = q + ((size_t)(b * (size_t)L + t0 + trow) * H + h) * DK;
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag fk, fq, fs;
                load_frag_f32(fk, Ks + trow * KP + 32 * kb + 8 * lq);
                if (trow < Lc) load_row8<TI>(fq, qrow + 32 * kb + 8 * lq);
                else zero_frag(fq);
                load_frag_f32(fs, St + (16 * J + lr) * KP + 32 * kb + 8 * lq);
                mma<PREC, true, false>(xk, fk, fs);
                mma<PREC, true, false>(xq, fq, fs);
            }
            float rr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + 4 * lq + r;
                const float eg = expf(gs[t]);
                const float vv = (t < Lc) ? load1<TI>(v + ((size_t)(b * (size_t)L + t0 + t) * H + h) * DV + v0 + 16 * J + lr) : 0.f;
                rr[r] = vv - eg * xk[r];
                Oacc[m][r] = eg * xq[r];
            }
            *reinterpret_cast<float4 *>(Rt + (16 * J + lr) * CP + 16 * I + 4 * lq) = make_float4(rr[0], rr[1], rr[2], rr[3]);
        }
        __syncthreads();

        // U = Tm R;  Ut = U, U2t = e^{g_C - g} U
        const float gC = gs[Lc - 1];
#pragma unroll
        for (int m = 0; m < MAXO; ++m) {
            const int o = wave + 4 * m;
            if (o >= NT_O) continue;
            const int I = o / NTV, J = o % NTV;
            f32x4 uacc = {0.f, 0.f, 0.f, 0.f};
            const int nkb = (16 * I + 16 + 31) / 32;
            for (int kb = 0; kb < nkb; ++kb) {
                const int kc = 32 * kb + 8 * lq;
                Frag fa, fb;
                if (kc < C) {
                    load_frag_f32(fa, Tg + (16 * I + lr) * C + kc);
                    load_frag_f32(fb, Rt + (16 * J + lr) * CP + kc);
                } else {
                    zero_frag(fa);
                    zero_frag(fb);
                }
                mma<PREC, false, false>(uacc, fa, fb);
            }
            float w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + 4 * lq + r;
                w[r] = expf(gC - gs[t]) * uacc[r];
            }
            *reinterpret_cast<float4 *>(Ut + (16 * J + lr) * CP + 16 * I + 4 * lq) = make_float4(uacc[0], uacc[1], uacc[2], uacc[3]);
            *reinterpret_cast<float4 *>(U2t + (16 * J + lr) * CP + 16 * I + 4 * lq) = make_float4(w[0], w[1], w[2], w[3]);
        }
        __syncthreads();

        // O += P U, store
#pragma unroll
        for (int m = 0; m < MAXO; ++m) {
            const int o = wave + 4 * m;
            if (o >= NT_O) continue;
            const int I = o / NTV, J = o % NTV;
            const int nkb = (16 * I + 16 + 31) / 32;
            for (int kb = 0; kb < nkb; ++kb) {
                const int kc = 32 * kb + 8 * lq;
                Frag fa, fb;
                if (kc < C) {
                    load_frag_f32(fa, Pg + (16 * I + lr) * C + kc);
                    load_frag_f32(fb, Ut + (16 * J + lr) * CP + kc);
                } else {
                    zero_frag(fa);
                    zero_frag(fb);
                }
                mma<PREC, false, false>(Oacc[m], fa, fb);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + 4 * lq + r;
                if (t < Lc) store1<TO>(out + ((size_t)(b * (size_t)L + t0 + t) * H + h) * DV + v0 + 16 * J + lr, Oacc[m][r]);
            }
        }

        // S <- e^{g_C} S + K^T U2
        const float eC = expf(gC);
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
            const int s = wave + 4 * m;
            if (s >= NT_S) continue;
            const int Ik = s / NTV, J = s % NTV;
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[m][r] *= eC;
#pragma unroll
            for (int kb = 0; kb < NKB_C; ++kb) {
                const int kc = 32 * kb + 8 * lq;
                Frag fa, fb;
                if (kc < C) {
                    load_frag_strided(fa, Ks + kc * KP + 16 * Ik + lr, KP);
                    load_frag_f32(fb, U2t + (16 * J + lr) * CP + kc);
                } else {
                    zero_frag(fa);
                    zero_frag(fb);
                }
                mma<PREC, true, false>(Sacc[m], fa, fb);
            }
            *reinterpret_cast<float4 *>(St + (16 * J + lr) * KP + 16 * Ik + 4 * lq) =
                make_float4(Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
        }
    }

    if (state_out) {
#pragma unroll
        for (int m = 0; m < MAXS; ++m) {
            const int s = wave + 4 * m;
            if (s >= NT_S) continue;
            const int Ik = s / NTV, J = s % NTV;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                state_out[(unit * DK + 16 * Ik + 4 * lq + r) * DV + v0 + 16 * J + lr] = Sacc[m][r];
        }
    }
}

size_t prefill_head_ws_bytes(int B, int L, int H, int C) {
    const size_t NC = (size_t)((L + C - 1) / C);
    return (size_t)B * H * NC * (size_t)(2 * C * C + C) * sizeof(float);
}

template <int D, int C, int PREC, typename TI, typename TO>
static hipError_t run(const GdnArgs &a, hipStream_t s) {
    constexpr int BV = 32;
    const int NC = (a.L + C - 1) / C;
    hipLaunchKernelGGL((prep_head_kernel<D, C, PREC, TI>), dim3(NC, a.H, a.B), dim3(256), 0, s,
                       (const TI *)a.q, (const TI *)a.k, a.alpha, a.beta, (float *)a.ws, a.L, a.H, NC);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_head_kernel<D, D, BV, C, PREC, TI, TO>), dim3(D / BV, a.H, a.B), dim3(256), 0, s,
                       (const TI *)a.q, (const TI *)a.k, (const TI *)a.v, (const float *)a.ws, a.state_in,
                       (TO *)a.out, a.state_out, a.L, a.H, NC);
    return hipGetLastError();
}

template <int D, int C>
static hipError_t run_t(const GdnArgs &a, hipStream_t s) {
    if (a.qkv_bf16)
        return a.out_bf16 ? run<D, C, PREC_BF16, uint16_t, uint16_t>(a, s) : run<D, C, PREC_BF16, uint16_t, float>(a, s);
    return a.out_bf16 ? run<D, C, PREC_F32, float, uint16_t>(a, s) : run<D, C, PREC_F32, float, float>(a, s);
}

template <int D>
static hipError_t run_c(const GdnArgs &a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return run_t<D, 16>(a, s);
        case 32: return run_t<D, 32>(a, s);
        default: return run_t<D, 64>(a, s);
    }
}

hipError_t launch_prefill_head(const GdnArgs &a, hipStream_t s) {
    return a.dk == 64 ? run_c<64>(a, s) : run_c<128>(a, s);
}

}  // namespace lt2
