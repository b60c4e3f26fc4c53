// bwd_channel.hip -- backward pass of the gated delta rule with a per-channel
// gate (KDA form, alpha_t in R^{d_k}), token by token in fp32.
//
// Forward (LT2 explainer, paithon.it, "Sostituire il motore", state-update
// equation, read out o_t = S_t^T q_t), with D_t = Diag(alpha_t):
//   y_t = S_{t-1}^T k_t,  E_t = S_{t-1} - beta_t k_t y_t^T,
//   S_t = D_t E_t + beta_t k_t v_t^T,  o_t = S_t^T q_t.
// Reverse mode for a loss with cotangents dO (outputs) and dS_L (final state),
// G_t the cotangent of S_t (G_L = dS_L), walking t = L .. 1:
//   G_t  += q_t dO_t^T                       dq_t = S_t dO_t
//   d(log alpha_t)_i = alpha_ti sum_j G_t,ij E_t,ij
//   dE = D_t G_t,   z = dE^T k_t,            dv_t = beta_t G_t^T k_t
//   dbeta_t = k_t^T G_t v_t - k_t^T dE y_t
//   dk_t = beta_t (G_t v_t - S_{t-1} z - dE y_t)
//   G_{t-1} = dE - beta_t k_t z^T            dS_0 = G_0
// Columns of S and of G evolve independently (column j only sees v_j, dO_j), so
// the work splits over column blocks; the row quantities dq, dk, d(log alpha)
// and dbeta sum over all columns.
//
// One workgroup of 8 waves per (b, h, 16-column block); each wave owns two
// state columns and every row (lane l: rows RPL l .. RPL l + RPL - 1, RPL =
// d/64), so sums over rows are wave reductions in registers (DPP and row
// swaps) and sums over the wave's columns stay in its lanes.  The workgroup
// first runs the recurrence forward and stores the state entering every
// segment of 16 tokens.  Then, for the segments in reverse order and each
// segment's two halves of 8 tokens (second half first), it recomputes the
// half's 9 states into registers from the segment's checkpoint and walks its
// tokens backwards, keeping the row quantities of its columns in registers;
// the eight waves' sums are then added through LDS (one write and one read per
// value) and written to a partial buffer per column block, which a second
// kernel sums.  Inputs of a segment are staged in LDS as fp32 with 16-byte
// loads issued one segment ahead.
#include "common.h"
#include "internal.h"

namespace lt2 {

namespace {

constexpr int KS = 16;               // segment (checkpoint interval) in tokens
constexpr int HS = KS / 2;           // tokens per backward half-segment
constexpr int KCOL = 2;              // state columns per wave
constexpr int KW = 8;                // waves per workgroup
constexpr int KBV = KCOL * KW;       // columns per workgroup
constexpr int KNT = 64 * KW;

struct KdaLayout {
    size_t ck, part, total;          // byte offsets: checkpoints, row partials
};

KdaLayout kda_layout(int B, int L, int H, int d) {
    const size_t units = (size_t)B * H, NS = (size_t)(L + KS - 1) / KS, ncb = (size_t)d / KBV;
    const size_t n_tok = (size_t)B * L * H;
    KdaLayout w{};
    w.ck = 0;
    w.part = units * NS * (size_t)d * d * 4;
    w.total = w.part + ncb * (3 * n_tok * (size_t)d + n_tok) * 4;
    return w;
}

// Sum over the 64 lanes, in registers: DPP within rows of 16 lanes (pairs,
// quads, mirrored half rows, mirrored rows), then the row-swap permutes.
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dppf<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dppf<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dppf<0x141>(x);   // row_half_mirror
    x += dppf<0x140>(x);   // row_mirror
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// KCOL consecutive floats (8- or 16-byte aligned)
__device__ __forceinline__ void ld_cols(const float *p, float (&x)[KCOL]) {
#pragma unroll
    for (int j = 0; j < KCOL; j += 2) {
        const float2 t = *reinterpret_cast<const float2 *>(p + j);
        x[j] = t.x;
        x[j + 1] = t.y;
    }
}
__device__ __forceinline__ void st_cols(float *p, const float (&x)[KCOL]) {
#pragma unroll
    for (int j = 0; j < KCOL; j += 2) *reinterpret_cast<float2 *>(p + j) = make_float2(x[j], x[j + 1]);
}

// 16 bytes of T -> fp32 values (8 bf16 or 4 fp32)
template <typename T>
struct Piece {
    static constexpr int N = 16 / (int)sizeof(T);
};
__device__ __forceinline__ void widen(const u32x4 u, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void widen(const u32x4 u, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(u[i]);
}

template <int D, typename TI, typename TO>
__global__ __launch_bounds__(KNT) void kda_bwd_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                       const TI *__restrict__ v, const float *__restrict__ alpha,
                                                       const float *__restrict__ beta, const float *state_in,
                                                       const TO *__restrict__ dout, const float *dstate_out,
                                                       float *__restrict__ dv_out, float *dstate_in,
                                                       float *__restrict__ ck, float *__restrict__ part, int B, int L,
                                                       int H) {
    constexpr int RPL = D / 64;                  // rows per lane
    constexpr int NCB = D / KBV;
    constexpr int EI = Piece<TI>::N, EO = Piece<TO>::N;
    constexpr int PK = KS * D / EI;              // 16-byte pieces of a segment's k (and q)
    constexpr int PA = KS * D / 4;               // ... of its alpha
    constexpr int PV = KS * KBV / EI;            // ... of the block's v columns
    constexpr int PD = KS * KBV / EO;            // ... of the block's dO columns
    constexpr int NPK = (PK + KNT - 1) / KNT, NPA = (PA + KNT - 1) / KNT;
    static_assert(PV + PD + KS / 4 <= KNT, "one small piece per thread");
    __shared__ __attribute__((aligned(16))) float sk[2][KS][D], sq[2][KS][D], sa[2][KS][D];
    __shared__ __attribute__((aligned(16))) float sv[2][KS][KBV], sd[2][KS][KBV], sb[2][KS];
    __shared__ float red[KW][HS][3][D];          // each wave's row sums of a half-segment: dq, dk, d(log alpha)
    __shared__ float redb[KW][HS];               // ... and its dbeta

    const int cb = blockIdx.x % NCB;
    const size_t unit = blockIdx.x / NCB;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cw = KCOL * wave;                  // this wave's first column inside the block
    const int c0 = cb * KBV + cw;                // ... in the state
    const int r0 = RPL * lane;                   // this lane's first row
    const int NS = (L + KS - 1) / KS;
    const size_t n_tok = (size_t)B * L * H;
    float *ckp = ck + unit * (size_t)NS * D * D;

    auto tok_of = [&](int t) __attribute__((always_inline)) { return ((size_t)b * L + t) * H + h; };

    // ---- segment inputs: 16-byte loads into registers, then fp32 into LDS ----
    // (tokens past L: k = q = 0, alpha = 1, beta = 0, v = dO = 0)
    u32x4 rk[NPK], rq[NPK], ra[NPA], rvd = {};
    auto fetch = [&](int s) __attribute__((always_inline)) {
        const int t0 = s * KS;
#pragma unroll
        for (int m = 0; m < NPK; ++m) {
            const int p = min(tid + KNT * m, PK - 1);
            const int tt = p / (D / EI), c = (p % (D / EI)) * EI;
            const size_t o = tok_of(min(t0 + tt, L - 1)) * D + c;
            rk[m] = *reinterpret_cast<const u32x4 *>(k + o);
            rq[m] = *reinterpret_cast<const u32x4 *>(q + o);
        }
#pragma unroll
        for (int m = 0; m < NPA; ++m) {
            const int p = min(tid + KNT * m, PA - 1);
            const int tt = p / (D / 4), c = (p % (D / 4)) * 4;
            ra[m] = *reinterpret_cast<const u32x4 *>(alpha + tok_of(min(t0 + tt, L - 1)) * D + c);
        }
        if (tid < PV) {
            const int tt = tid / (KBV / EI), c = (tid % (KBV / EI)) * EI;
            rvd = *reinterpret_cast<const u32x4 *>(v + tok_of(min(t0 + tt, L - 1)) * D + cb * KBV + c);
        } else if (tid < PV + PD) {
            const int p = tid - PV, tt = p / (KBV / EO), c = (p % (KBV / EO)) * EO;
            rvd = *reinterpret_cast<const u32x4 *>(dout + tok_of(min(t0 + tt, L - 1)) * D + cb * KBV + c);
        } else if (tid < PV + PD + KS / 4) {
            const int p = tid - PV - PD;
#pragma unroll
            for (int e = 0; e < 4; ++e) rvd[e] = __float_as_uint(beta[tok_of(min(t0 + 4 * p + e, L - 1))]);
        }
    };
    auto stage = [&](int s, int buf) __attribute__((always_inline)) {
        const int t0 = s * KS;
#pragma unroll
        for (int m = 0; m < NPK; ++m) {
            const int p = tid + KNT * m;
            if (p < PK) {
                const int tt = p / (D / EI), c = (p % (D / EI)) * EI;
                const bool ok = t0 + tt < L;
                float fk[EI], fq[EI];
                widen(rk[m], fk);
                widen(rq[m], fq);
#pragma unroll
                for (int e = 0; e < EI; ++e) {
                    sk[buf][tt][c + e] = ok ? fk[e] : 0.f;
                    sq[buf][tt][c + e] = ok ? fq[e] : 0.f;
                }
            }
        }
#pragma unroll
        for (int m = 0; m < NPA; ++m) {
            const int p = tid + KNT * m;
            if (p < PA) {
                const int tt = p / (D / 4), c = (p % (D / 4)) * 4;
                const bool ok = t0 + tt < L;
#pragma unroll
                for (int e = 0; e < 4; ++e) sa[buf][tt][c + e] = ok ? __uint_as_float(ra[m][e]) : 1.f;
            }
        }
        if (tid < PV) {
            const int tt = tid / (KBV / EI), c = (tid % (KBV / EI)) * EI;
            const bool ok = t0 + tt < L;
            float f[EI];
            widen(rvd, f);
#pragma unroll
            for (int e = 0; e < EI; ++e) sv[buf][tt][c + e] = ok ? f[e] : 0.f;
        } else if (tid < PV + PD) {
            const int p = tid - PV, tt = p / (KBV / EO), c = (p % (KBV / EO)) * EO;
            const bool ok = t0 + tt < L;
            float f[EO];
            widen(rvd, f);
#pragma unroll
            for (int e = 0; e < EO; ++e) sd[buf][tt][c + e] = ok ? f[e] : 0.f;
        } else if (tid < PV + PD + KS / 4) {
            const int p = tid - PV - PD;
#pragma unroll
            for (int e = 0; e < 4; ++e) sb[buf][4 * p + e] = (t0 + 4 * p + e < L) ? __uint_as_float(rvd[e]) : 0.f;
        }
    };
    // One forward token on the wave's state columns; y = S^T k of the old state.
    auto step = [&](float (&S)[RPL][KCOL], float (&y)[KCOL], int buf, int tt) __attribute__((always_inline)) {
        float kr[RPL], ar[RPL];
#pragma unroll
        for (int i = 0; i < RPL; ++i) { kr[i] = sk[buf][tt][r0 + i]; ar[i] = sa[buf][tt][r0 + i]; }
        const float bt = sb[buf][tt];
        float v4[KCOL];
        ld_cols(&sv[buf][tt][cw], v4);
#pragma unroll
        for (int j = 0; j < KCOL; ++j) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) p += kr[i] * S[i][j];
            y[j] = wave_sum(p);
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const float bk = bt * kr[i];
#pragma unroll
            for (int j = 0; j < KCOL; ++j) S[i][j] = ar[i] * (S[i][j] - bk * y[j]) + bk * v4[j];
        }
    };

    // ---- forward: the state entering every segment ----
    float S[RPL][KCOL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int j = 0; j < KCOL; ++j) S[i][j] = state_in ? state_in[(unit * D + r0 + i) * D + c0 + j] : 0.f;
    fetch(0);
    stage(0, 0);
    __syncthreads();
    for (int s = 0; s < NS; ++s) {
        const int buf = s & 1;
        if (s + 1 < NS) fetch(s + 1);
#pragma unroll
        for (int i = 0; i < RPL; ++i) st_cols(&ckp[((size_t)s * D + r0 + i) * D + c0], S[i]);
        const int n = min(KS, L - s * KS);
        for (int tt = 0; tt < n; ++tt) {
            float y[KCOL];
            step(S, y, buf, tt);
        }
        if (s + 1 < NS) stage(s + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- backward, segments in reverse, each in two halves (second half first) ----
    float G[RPL][KCOL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int j = 0; j < KCOL; ++j) G[i][j] = dstate_out ? dstate_out[(unit * D + r0 + i) * D + c0 + j] : 0.f;
    fetch(NS - 1);
    stage(NS - 1, 0);
    __syncthreads();
    float *pb = part + (size_t)cb * (3 * n_tok * D + n_tok);
    for (int jseg = 0; jseg < NS; ++jseg) {
        const int s = NS - 1 - jseg, buf = jseg & 1;
        const int t0 = s * KS;
        const int n = min(KS, L - t0);
        if (s > 0) fetch(s - 1);
        for (int half = 1; half >= 0; --half) {
            const int u0 = HS * half;             // first token of the half inside the segment
            const int nh = min(HS, n - u0);       // its tokens (may be <= 0 for a ragged last segment)
            if (nh > 0) {
                // the state entering the half: the checkpoint advanced by u0 tokens
                float Sx[HS + 1][RPL][KCOL], yy[HS][KCOL];
#pragma unroll
                for (int i = 0; i < RPL; ++i) ld_cols(&ckp[((size_t)s * D + r0 + i) * D + c0], Sx[0][i]);
                for (int tt = 0; tt < u0; ++tt) {
                    float y[KCOL];
                    step(Sx[0], y, buf, tt);
                }
#pragma unroll
                for (int u = 0; u < HS; ++u) {
#pragma unroll
                    for (int i = 0; i < RPL; ++i)
#pragma unroll
                        for (int j = 0; j < KCOL; ++j) Sx[u + 1][i][j] = Sx[u][i][j];
#pragma unroll
                    for (int j = 0; j < KCOL; ++j) yy[u][j] = 0.f;
                    if (u < nh) step(Sx[u + 1], yy[u], buf, u0 + u);
                }
                float rq_[HS][RPL], rk_[HS][RPL], ra_[HS][RPL], rb_[HS];
#pragma unroll
                for (int u = HS - 1; u >= 0; --u) {
                    if (u >= nh) {
#pragma unroll
                        for (int i = 0; i < RPL; ++i) { rq_[u][i] = 0.f; rk_[u][i] = 0.f; ra_[u][i] = 0.f; }
                        rb_[u] = 0.f;
                        continue;
                    }
                    const int tt = u0 + u;
                    float kr[RPL], qr[RPL], ar[RPL];
#pragma unroll
                    for (int i = 0; i < RPL; ++i) {
                        kr[i] = sk[buf][tt][r0 + i]; qr[i] = sq[buf][tt][r0 + i]; ar[i] = sa[buf][tt][r0 + i];
                    }
                    float v4[KCOL], d4[KCOL];
                    ld_cols(&sv[buf][tt][cw], v4);
                    ld_cols(&sd[buf][tt][cw], d4);
                    const float bt = sb[buf][tt];
                    float dE[RPL][KCOL], zp[KCOL], gkp[KCOL], dbp = 0.f;
#pragma unroll
                    for (int j = 0; j < KCOL; ++j) { zp[j] = 0.f; gkp[j] = 0.f; }
#pragma unroll
                    for (int i = 0; i < RPL; ++i) {
                        float dq_ = 0.f, dla = 0.f, gv = 0.f, dey = 0.f;
#pragma unroll
                        for (int j = 0; j < KCOL; ++j) {
                            G[i][j] += qr[i] * d4[j];
                            dq_ += Sx[u + 1][i][j] * d4[j];
                            // E = S_{t-1} - beta k y: exact zero gradient for alpha = 0 and
                            // no cancellation for small alpha (unlike S_t - beta k v = alpha E)
                            dla += G[i][j] * (Sx[u][i][j] - bt * kr[i] * yy[u][j]);
                            dE[i][j] = ar[i] * G[i][j];
                            gv += G[i][j] * v4[j];
                            dey += dE[i][j] * yy[u][j];
                            zp[j] += dE[i][j] * kr[i];
                            gkp[j] += G[i][j] * kr[i];
                        }
                        rq_[u][i] = dq_;
                        ra_[u][i] = ar[i] * dla;
                        rk_[u][i] = gv - dey;             // the S_{t-1} z term is added below
                        dbp += kr[i] * (gv - dey);
                    }
                    float z[KCOL], gk[KCOL];
#pragma unroll
                    for (int j = 0; j < KCOL; ++j) { z[j] = wave_sum(zp[j]); gk[j] = wave_sum(gkp[j]); }
                    rb_[u] = wave_sum(dbp);
#pragma unroll
                    for (int i = 0; i < RPL; ++i) {
                        float sz = 0.f;
#pragma unroll
                        for (int j = 0; j < KCOL; ++j) {
                            sz += Sx[u][i][j] * z[j];
                            G[i][j] = dE[i][j] - bt * kr[i] * z[j];
                        }
                        rk_[u][i] = bt * (rk_[u][i] - sz);
                    }
                    if (lane < KCOL) {
                        float g = gk[0];
#pragma unroll
                        for (int j = 1; j < KCOL; ++j) g = lane == j ? gk[j] : g;
                        dv_out[tok_of(t0 + tt) * D + c0 + lane] = bt * g;
                    }
                }
                // this wave's row sums of the half -> LDS
#pragma unroll
                for (int u = 0; u < HS; ++u) {
#pragma unroll
                    for (int i = 0; i < RPL; ++i) {
                        red[wave][u][0][r0 + i] = rq_[u][i];
                        red[wave][u][1][r0 + i] = rk_[u][i];
                        red[wave][u][2][r0 + i] = ra_[u][i];
                    }
                    if (lane == 0) redb[wave][u] = rb_[u];
                }
            }
            __syncthreads();
            // the waves' sums of the half -> this block's partial buffer
            if (nh > 0) {
                for (int idx = tid; idx < nh * 3 * D; idx += KNT) {
                    const int u = idx / (3 * D), rem = idx % (3 * D), qd = rem / D, c = rem % D;
                    float sum = 0.f;
#pragma unroll
                    for (int w = 0; w < KW; ++w) sum += red[w][u][qd][c];
                    pb[(size_t)qd * n_tok * D + tok_of(t0 + u0 + u) * D + c] = sum;
                }
                if (tid < nh) {
                    float sum = 0.f;
#pragma unroll
                    for (int w = 0; w < KW; ++w) sum += redb[w][tid];
                    pb[3 * n_tok * D + tok_of(t0 + u0 + tid)] = sum;
                }
            }
            __syncthreads();
        }
        if (s > 0) stage(s - 1, buf ^ 1);
        __syncthreads();
    }
    if (dstate_in) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) st_cols(&dstate_in[(unit * D + r0 + i) * D + c0], G[i]);
    }
}

// dq, dk, d(log alpha) [n_tok, D] and dbeta [n_tok] = sums of the column-block partials.
__global__ __launch_bounds__(256) void kda_bwd_reduce_kernel(const float *__restrict__ part, int ncb, size_t n_tok,
                                                             int D, float *__restrict__ dq, float *__restrict__ dk,
                                                             float *__restrict__ dla, float *__restrict__ dbeta) {
    const size_t n_row = n_tok * (size_t)D, stride = 3 * n_row + n_tok;
    const size_t total = 3 * n_row + n_tok;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int c = 0; c < ncb; ++c) s += part[(size_t)c * stride + i];
        if (i < n_row) dq[i] = s;
        else if (i < 2 * n_row) dk[i - n_row] = s;
        else if (i < 3 * n_row) dla[i - 2 * n_row] = s;
        else dbeta[i - 3 * n_row] = s;
    }
}

// The same sums four elements at a time when the token count is a multiple of
// four (every partial buffer then starts 16-byte aligned and no group of four
// straddles two outputs): 16-byte non-temporal loads (each partial is read
// once), all NCB of an element group in flight, added in the same order as
// above, so the results are bit-identical.
template <int NCB>
__global__ __launch_bounds__(256) void kda_bwd_reduce4_kernel(const float *__restrict__ part, size_t n_tok, int D,
                                                              float *__restrict__ dq, float *__restrict__ dk,
                                                              float *__restrict__ dla, float *__restrict__ dbeta) {
    const size_t n_row = n_tok * (size_t)D, stride4 = (3 * n_row + n_tok) / 4;
    const f32x4 *p4 = reinterpret_cast<const f32x4 *>(part);
    for (size_t i4 = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i4 < stride4; i4 += (size_t)gridDim.x * blockDim.x) {
        f32x4 x[NCB];
#pragma unroll
        for (int c = 0; c < NCB; ++c) x[c] = __builtin_nontemporal_load(p4 + (size_t)c * stride4 + i4);
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCB; ++c) sum += x[c];
        const size_t i = 4 * i4;
        float *dst = i < n_row ? dq + i : (i < 2 * n_row ? dk + (i - n_row)
                                                            : (i < 3 * n_row ? dla + (i - 2 * n_row) : dbeta + (i - 3 * n_row)));
        *reinterpret_cast<f32x4 *>(dst) = sum;
    }
}

template <int D, typename TI, typename TO>
hipError_t run_kda(const GdnBwdArgs &a, hipStream_t s) {
    const KdaLayout w = kda_layout(a.B, a.L, a.H, D);
    unsigned char *ws = static_cast<unsigned char *>(a.ws);
    float *ck = reinterpret_cast<float *>(ws + w.ck);
    float *part = reinterpret_cast<float *>(ws + w.part);
    const unsigned units = (unsigned)a.B * (unsigned)a.H;
    hipLaunchKernelGGL((kda_bwd_kernel<D, TI, TO>), dim3(units * (D / KBV)), dim3(KNT), 0, s, (const TI *)a.q,
                       (const TI *)a.k, (const TI *)a.v, a.alpha, a.beta, a.state_in, (const TO *)a.dout,
                       a.dstate_out, a.dv, a.dstate_in, ck, part, a.B, a.L, a.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n_tok = (size_t)a.B * a.L * a.H;
    const size_t total = 3 * n_tok * D + n_tok;
    // the vector form needs 16-byte aligned outputs too (the row gradients are)
    const bool vec = n_tok % 4 == 0 && ((uintptr_t)a.dq | (uintptr_t)a.dk | (uintptr_t)a.dlog_alpha |
                                        (uintptr_t)a.dbeta) % 16 == 0;
    if (vec) {
        const size_t total4 = total / 4;
        const unsigned blocks = (unsigned)((total4 + 255) / 256 < 65536 ? (total4 + 255) / 256 : 65536);
        hipLaunchKernelGGL((kda_bwd_reduce4_kernel<D / KBV>), dim3(blocks), dim3(256), 0, s, part, n_tok, D, a.dq,
                           a.dk, a.dlog_alpha, a.dbeta);
    } else {
        const unsigned blocks = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
        hipLaunchKernelGGL(kda_bwd_reduce_kernel, dim3(blocks), dim3(256), 0, s, part, D / KBV, n_tok, D, a.dq, a.dk,
                           a.dlog_alpha, a.dbeta);
    }
    return hipGetLastError();
}

template <int D>
hipError_t run_kda_t(const GdnBwdArgs &a, hipStream_t s) {
    if (a.qkv_bf16)
        return a.dout_bf16 ? run_kda<D, uint16_t, uint16_t>(a, s) : run_kda<D, uint16_t, float>(a, s);
    return a.dout_bf16 ? run_kda<D, float, uint16_t>(a, s) : run_kda<D, float, float>(a, s);
}

}  // namespace

size_t kda_bwd_ws_bytes(int B, int L, int H, int d) { return kda_layout(B, L, H, d).total; }

hipError_t launch_kda_bwd(const GdnBwdArgs &a, hipStream_t s) {
    return a.d == 64 ? run_kda_t<64>(a, s) : run_kda_t<128>(a, s);
}

}  // namespace lt2
