// bwd.hip -- backward pass of the chunked gated delta rule, scalar gate.
//
// The forward recurrence (LT2 explainer, paithon.it, section "Sostituire il
// motore", the state-update equation, read out o_t = S_t^T q_t) in its chunk
// form, for one chunk of C tokens with S the state entering it:
//   g_t  = sum_{j<=t} log2 alpha_j (chunk-relative), gamma_t = 2^g_t,
//   Gam_ti = 2^(g_t - g_i) (i <= t), gamma_C = gamma of the chunk's last token
//   A = strict_lower(beta_t (k_t . k_i) Gam_ti),  N = (I + A)^-1,  Tm = N diag(beta)
//   P = lower_incl((q_t . k_i) Gam_ti)
//   R = V - diag(gamma) K S,   U = Tm R
//   O = diag(gamma) Q S + P U,   S' = gamma_C S + K^T diag(gamma_C / gamma) U
// Its reverse-mode derivative for a loss with output cotangent dO and cotangent
// dS' of the state leaving the chunk:
//   dU = P^T dO + diag(gamma_C / gamma) K dS'      dR = diag(beta) N^T dU = dV
//   dS = Q^T diag(gamma) dO + gamma_C dS' - K^T diag(gamma) dR      (to the previous chunk)
//   dP = (dO U^T) o lower_incl,  dTm = dU R^T,  dA = -N^T (dTm diag(beta)) N^T  (strict lower)
//   dQ = diag(gamma) dO S^T + (dP o Gam) K
//   dK = (dP o Gam)^T Q + diag(gamma_C/gamma) U dS'^T - diag(gamma) dR S^T + E K + E^T K,
//        E_ti = dA_ti beta_t Gam_ti
//   dbeta_t = sum_s dTm_st N_st + sum_i dA_ti (k_t . k_i) Gam_ti
// and, for the natural-log cumulative gate Gn_t (gamma_t = e^Gn_t):
//   d(log alpha_j) = sum_{t >= j} (gq_t + gk_t) + sum_{t < j} gd_t
//                    + sum_{t >= j} sum_{i < j} X_ti + gamma_C <dS', S>
// with gq_t = gamma_t <dO_t, (Q S)_t>, gk_t = -gamma_t <dR_t, (K S)_t>,
// gd_t = (gamma_C/gamma_t) <U_t, (K dS')_t> and X = dP o P + dA o A: gamma_t
// depends on the gates up to t, gamma_C/gamma_t on those after t, and Gam_ti on
// those in (i, t].  (Summing per-token derivatives and then a suffix sum would
// add and cancel the pairs with i >= j, which loses the small gradient of a
// fast-decaying gate in fp32.)
//
// The chunk-relative cumulative log2 gates are kept in fp64: with a fast decay
// they reach hundreds of octaves inside a chunk, where an fp32 sum would leave
// every decay 2^(g_t - g_i) between nearby tokens with a relative error of
// |g| 2^-24; each decay is formed from an fp64 difference and then
// exponentiated in fp32.
//
// Four launches, all fp32 arithmetic apart from those sums (bf16 inputs are
// widened exactly):
//   bwd_prep_kernel    one workgroup per (b, h, chunk): g, N, P into the workspace
//   bwd_states_kernel  one per (b, h, 32-column block): the state entering every chunk
//   bwd_dstate_kernel  one per (b, h, 32-column block), chunks in reverse: the
//                      cotangent of the state leaving every chunk, and dS_0
//   bwd_grads_kernel   one per (b, h, chunk): dv, dq, dk, dbeta, d(log alpha)
// Products run on the fp32 matrix cores (v_mfma_f32_16x16x4f32: exact fp32
// products, fp32 sums) from LDS operands; each wave owns 16-row output tiles.
// Every load of a chunk is issued before the first of them is used.
#include "common.h"
#include "internal.h"

namespace lt2 {

namespace {

constexpr int BC = 64;        // chunk length of the backward pass
constexpr int BNT = 256;      // threads per workgroup
constexpr int CPp = BC + 1;   // pitch of C x C matrices (odd: conflict-free column reads)

struct BwdLayout {
    size_t gnp, s, ds, total;   // byte offsets of the g/N/P, state and state-cotangent regions
};

// per (unit, chunk): g [C] fp64, then N, P [C][C] fp32
constexpr size_t G_FLOATS = 2 * BC;
constexpr size_t GNP_FLOATS = G_FLOATS + 2 * BC * BC;

BwdLayout bwd_layout(int B, int L, int H, int d) {
    const size_t units = (size_t)B * H, NC = (size_t)(L + BC - 1) / BC;
    BwdLayout w{};
    w.gnp = 0;
    w.s = w.gnp + units * NC * GNP_FLOATS * 4;
    w.ds = w.s + units * NC * (size_t)d * d * 4;
    w.total = w.ds + units * NC * (size_t)d * d * 4;
    return w;
}

// Rows [t0, t0 + n) of a [.., H, W] tensor (token stride tok) into LDS dst
// [BC][pitch] as fp32, 16 bytes per load; rows >= n are zero.  Rows start
// 16-byte aligned (aligned base, W a multiple of 16 bytes).  fetch() issues
// every load of the tile into registers, put() widens and stores them, so a
// caller can issue several tiles' loads before the first wait.
__device__ __forceinline__ void widen16(float *d, u32x4 x, const uint16_t *) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d[2 * i] = __uint_as_float(x[i] << 16);
        d[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void widen16(float *d, u32x4 x, const float *) {
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = __uint_as_float(x[i]);
}
template <int W, typename T>
struct Rows {
    static constexpr int VEC = 16 / (int)sizeof(T), PR = W / VEC, IT = (BC * PR + BNT - 1) / BNT;
    u32x4 x[IT];
    __device__ __forceinline__ void fetch(const T *src, size_t tok, int n) {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int idx = threadIdx.x + BNT * i, r = idx / PR, c = VEC * (idx % PR);
            x[i] = u32x4{0u, 0u, 0u, 0u};
            if (idx < BC * PR && r < n) x[i] = *reinterpret_cast<const u32x4 *>(src + (size_t)r * tok + c);
        }
    }
    __device__ __forceinline__ void put(float *dst, int pitch) const {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int idx = threadIdx.x + BNT * i, r = idx / PR, c = VEC * (idx % PR);
            if (idx < BC * PR) widen16(dst + r * pitch + c, x[i], static_cast<const T *>(nullptr));
        }
    }
};
// A C x C fp32 matrix of the workspace (16-byte aligned, row-major) into LDS
// with pitch CPp, four 16-byte loads per thread.
struct CCm {
    static constexpr int IT = BC * BC / 4 / BNT;
    u32x4 x[IT];
    __device__ __forceinline__ void fetch(const float *src) {
#pragma unroll
        for (int i = 0; i < IT; ++i) x[i] = reinterpret_cast<const u32x4 *>(src)[threadIdx.x + BNT * i];
    }
    __device__ __forceinline__ void put(float *dst) const {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = 4 * (threadIdx.x + BNT * i), r = e / BC, c = e % BC;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[r * CPp + c + j] = __uint_as_float(x[i][j]);
        }
    }
};

// Chunk-relative inclusive prefix sums (fp64) of log2 alpha for tokens
// [t0, t0 + n); entries >= n repeat the last sum.  Computed by wave 0.
__device__ __forceinline__ void gate_prefix(double *g, const float *alpha, size_t gstride, int n) {
    if (threadIdx.x < 64) {
        const int l = threadIdx.x;
        double x = l < n ? (double)log2_gate(alpha[(size_t)l * gstride]) : 0.0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(x, o);
            if (l >= o) x += y;
        }
        g[l] = x;
    }
}

// 2^(a - b) from fp64 exponents
__device__ __forceinline__ float dexp2(double a, double b) { return exp2_fast((float)(a - b)); }

// ---------------------------------------------------------------------------
// g, N = (I + A)^-1 and P of one chunk.
template <int D, typename TI>
__global__ __launch_bounds__(BNT) void bwd_prep_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                       const float *__restrict__ alpha,
                                                       const float *__restrict__ beta, float *__restrict__ gnp,
                                                       int L, int H, int NC) {
    constexpr int DP = D + 1;
    __shared__ float Ks[BC * DP], Qs[BC * DP], As[BC * CPp], Ns[BC * CPp], bt[BC];
    __shared__ double g[BC];
    const int c = blockIdx.x % NC;
    const size_t unit = blockIdx.x / NC;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const int t0 = c * BC, n = min(BC, L - t0);
    const size_t tok = (size_t)H * D;
    const size_t row0 = ((size_t)b * L + t0) * H + h;   // (b, t0, h) in [B, L, H]
    {
        Rows<D, TI> rk, rq;
        rk.fetch(k + row0 * D, tok, n);
        rq.fetch(q + row0 * D, tok, n);
        rk.put(Ks, DP);
        rq.put(Qs, DP);
    }
    gate_prefix(g, alpha + row0, H, n);
    if (threadIdx.x < BC) bt[threadIdx.x] = threadIdx.x < n ? beta[row0 + (size_t)threadIdx.x * H] : 0.f;
    __syncthreads();
    // K K^T and Q K^T on the fp32 matrix cores: wave w owns rows 16w .. 16w + 15
    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int R0 = 16 * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), ra = R0 + lr;
    float *out = gnp + (unit * NC + c) * GNP_FLOATS;
#pragma unroll
    for (int j = 0; j < BC / 16; ++j) {
        f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = kk;
#pragma unroll 8
        for (int k0 = 0; k0 < D; k0 += 4) {
            const float kb = Ks[(16 * j + lr) * DP + k0 + lq];
            kk = __builtin_amdgcn_mfma_f32_16x16x4f32(Ks[ra * DP + k0 + lq], kb, kk, 0, 0, 0);
            qk = __builtin_amdgcn_mfma_f32_16x16x4f32(Qs[ra * DP + k0 + lq], kb, qk, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = R0 + 4 * lq + r, s = 16 * j + lr;
            const float gam = dexp2(g[t], g[min(s, t)]);
            As[t * CPp + s] = s < t ? bt[t] * kk[r] * gam : 0.f;
            out[G_FLOATS + BC * BC + t * BC + s] = (s <= t && t < n) ? qk[r] * gam : 0.f;   // P
        }
    }
    if (threadIdx.x < BC) reinterpret_cast<double *>(out)[threadIdx.x] = g[threadIdx.x];
    __syncthreads();
    // N = (I + A)^-1, blocked by 16: the four diagonal blocks by row substitution
    // in wave 0 (lane j owns column j and reads only that column's earlier rows,
    // so no barrier is needed between rows), then the off-diagonal blocks one
    // block-distance at a time:
    //   N_ij = -N_ii sum_{k=j}^{i-1} A_ik N_kj   (i > j)
    for (int idx = threadIdx.x; idx < BC * BC; idx += BNT) Ns[(idx / BC) * CPp + idx % BC] = 0.f;
    __syncthreads();
    if (threadIdx.x < 64) {
        const int bb = threadIdx.x / 16, j = threadIdx.x;   // column j of diagonal block bb
        for (int r = 0; r < 16; ++r) {
            const int t = 16 * bb + r;
            float x = t == j ? 1.f : 0.f;
            for (int i = j; i < t; ++i) x = fmaf(-As[t * CPp + i], Ns[i * CPp + j], x);
            if (j <= t) Ns[t * CPp + j] = x;
        }
    }
    __syncthreads();
    __shared__ float Ws[BC * CPp];   // W_ij = sum_k A_ik N_kj for the current distance
    for (int dist = 1; dist < 4; ++dist) {
        // W blocks (i, j = i - dist): 16 x 16 each, (4 - dist) of them
        const int nb = 4 - dist;
        for (int idx = threadIdx.x; idx < nb * 256; idx += BNT) {
            const int blk = idx / 256, e = idx % 256, r = e / 16, cc = e % 16;
            const int bi = blk + dist, bj = blk;
            const int t = 16 * bi + r, jj = 16 * bj + cc;
            float x = 0.f;
            for (int kk = 16 * bj; kk < 16 * bi; ++kk) x = fmaf(As[t * CPp + kk], Ns[kk * CPp + jj], x);
            Ws[t * CPp + jj] = x;
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < nb * 256; idx += BNT) {
            const int blk = idx / 256, e = idx % 256, r = e / 16, cc = e % 16;
            const int bi = blk + dist, bj = blk;
            const int t = 16 * bi + r, jj = 16 * bj + cc;
            float x = 0.f;
            for (int kk = 16 * bi; kk <= t; ++kk) x = fmaf(Ns[t * CPp + kk], Ws[kk * CPp + jj], x);
            Ns[t * CPp + jj] = -x;
        }
        __syncthreads();
    }
    for (int idx = threadIdx.x; idx < BC * BC; idx += BNT)
        out[G_FLOATS + idx] = Ns[(idx / BC) * CPp + idx % BC];
}

// ---------------------------------------------------------------------------
// The state entering every chunk, per 32-column block of the value dimension.
template <int D, typename TI>
__global__ __launch_bounds__(BNT) void bwd_states_kernel(const TI *__restrict__ k, const TI *__restrict__ v,
                                                         const float *__restrict__ beta,
                                                         const float *__restrict__ state_in,
                                                         const float *__restrict__ gnp, float *__restrict__ sws,
                                                         int L, int H, int NC) {
    constexpr int BV = 32, DP = D + 1, VP = BV + 1;
    __shared__ float Ss[D * VP], Ks[BC * DP], Vs[BC * VP], Ns[BC * CPp], Rs[BC * VP], Us[BC * VP], bt[BC];
    __shared__ double g[BC];
    constexpr int NB = D / BV;
    // matrix-core roles (fp32 16 x 16 x 4 products): wave w owns token rows
    // 16w .. 16w + 15 of the C x 32 products and state rows SR0 .. SR0 + 16 NR - 1
    constexpr int NR = D / 64;
    static_assert(BNT == 256 && BC == 64 && BV == 32, "four waves, two 16-column tiles");
    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R0 = 16 * wv, ra = R0 + lr, SR0 = 16 * NR * wv;
    const int vb = blockIdx.x % NB;
    const size_t unit = blockIdx.x / NB;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const size_t tok = (size_t)H * D;
    for (int idx = threadIdx.x; idx < D * BV; idx += BNT) {
        const int r = idx / BV, cc = idx % BV;
        Ss[r * VP + cc] = state_in ? state_in[(unit * D + r) * D + vb * BV + cc] : 0.f;
    }
    // The loads of chunk c + 1 are issued once chunk c's inputs are in LDS and
    // land while chunk c computes.
    Rows<D, TI> rk;
    Rows<BV, TI> rv;
    CCm nm;
    double gv = 0.0;
    float bv = 0.f;
    auto fetch = [&](int c) {
        const int t0 = c * BC, n = min(BC, L - t0);
        const size_t row0 = ((size_t)b * L + t0) * H + h;
        const float *gc = gnp + (unit * NC + c) * GNP_FLOATS;
        rk.fetch(k + row0 * D, tok, n);
        rv.fetch(v + row0 * D + vb * BV, tok, n);
        nm.fetch(gc + G_FLOATS);
        if (threadIdx.x < BC) {
            gv = reinterpret_cast<const double *>(gc)[threadIdx.x];
            bv = threadIdx.x < n ? beta[row0 + (size_t)threadIdx.x * H] : 0.f;
        }
    };
    fetch(0);
    for (int c = 0; c < NC; ++c) {
        const int t0 = c * BC, n = min(BC, L - t0);
        __syncthreads();
        // the state entering chunk c
        float *so = sws + (unit * NC + c) * (size_t)D * D;
        for (int idx = threadIdx.x; idx < D * BV; idx += BNT) {
            const int r = idx / BV, cc = idx % BV;
            so[r * D + vb * BV + cc] = Ss[r * VP + cc];
        }
        rk.put(Ks, DP);
        rv.put(Vs, VP);
        nm.put(Ns);
        if (threadIdx.x < BC) {
            g[threadIdx.x] = gv;
            bt[threadIdx.x] = bv;
        }
        if (c + 1 < NC) fetch(c + 1);
        __syncthreads();
        const double gC = g[n - 1];
        {   // R' = diag(beta) (V - diag(gamma) K S)
            f32x4 p[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
#pragma unroll 8
            for (int k0 = 0; k0 < D; k0 += 4) {   // two partial sums per tile (even, odd k-steps)
                const int h2 = (k0 >> 2) & 1;
                const float ka = Ks[ra * DP + k0 + lq];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    p[h2][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, Ss[(k0 + lq) * VP + 16 * j + lr], p[h2][j], 0, 0, 0);
            }
            const f32x4 a[2] = {p[0][0] + p[1][0], p[0][1] + p[1][1]};
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = R0 + 4 * lq + r, o = t * VP + 16 * j + lr;
                    Rs[o] = bt[t] * (Vs[o] - dexp2(g[t], 0.0) * a[j][r]);
                }
        }
        __syncthreads();
        {   // U' = diag(gamma_C / gamma) N R'
            f32x4 p[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 4) {   // two partial sums per tile
                const int h2 = (k0 >> 2) & 1;
                const float na = Ns[ra * CPp + k0 + lq];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    p[h2][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(na, Rs[(k0 + lq) * VP + 16 * j + lr], p[h2][j], 0, 0, 0);
            }
            const f32x4 a[2] = {p[0][0] + p[1][0], p[0][1] + p[1][1]};
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = R0 + 4 * lq + r;
                    Us[t * VP + 16 * j + lr] = dexp2(gC, g[t]) * a[j][r];
                }
        }
        __syncthreads();
        {   // S = gamma_C S + K^T U'  (wave w: state rows 16 (w NR + x) .., both column tiles)
            f32x4 a[NR][2];
#pragma unroll
            for (int x = 0; x < NR; ++x) a[x][0] = a[x][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k0 = 0; k0 < BC; k0 += 4) {
                const int kk = k0 + lq;
                const float u0 = Us[kk * VP + lr], u1 = Us[kk * VP + 16 + lr];
#pragma unroll
                for (int x = 0; x < NR; ++x) {
                    const float kt = Ks[kk * DP + SR0 + 16 * x + lr];
                    a[x][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt, u0, a[x][0], 0, 0, 0);
                    a[x][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt, u1, a[x][1], 0, 0, 0);
                }
            }
            const float gam = dexp2(gC, 0.0);
#pragma unroll
            for (int x = 0; x < NR; ++x)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float &y = Ss[(SR0 + 16 * x + 4 * lq + r) * VP + 16 * j + lr];
                        y = fmaf(gam, y, a[x][j][r]);
                    }
        }
    }
}

// ---------------------------------------------------------------------------
// Chunks in reverse: the cotangent of the state leaving every chunk (stored) and
// finally that of S_0.
template <int D, typename TI, typename TO>
__global__ __launch_bounds__(BNT) void bwd_dstate_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                         const TO *__restrict__ dout, const float *__restrict__ beta,
                                                         const float *__restrict__ dstate_out,
                                                         const float *__restrict__ gnp, float *__restrict__ dsws,
                                                         float *__restrict__ dstate_in, int L, int H, int NC) {
    constexpr int BV = 32, DP = D + 1, VP = BV + 1;
    __shared__ float dS[D * VP], Ks[BC * DP], Qs[BC * DP], dOs[BC * VP], Ns[BC * CPp], Ps[BC * CPp], dUs[BC * VP],
        dRs[BC * VP], bt[BC];
    __shared__ double g[BC];
    constexpr int NB = D / BV;
    // matrix-core roles as in the chunk-state kernel
    constexpr int NR = D / 64;
    static_assert(BNT == 256 && BC == 64 && BV == 32, "four waves, two 16-column tiles");
    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R0 = 16 * wv, ra = R0 + lr, SR0 = 16 * NR * wv;
    const int vb = blockIdx.x % NB;
    const size_t unit = blockIdx.x / NB;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const size_t tok = (size_t)H * D;
    for (int idx = threadIdx.x; idx < D * BV; idx += BNT) {
        const int r = idx / BV, cc = idx % BV;
        dS[r * VP + cc] = dstate_out ? dstate_out[(unit * D + r) * D + vb * BV + cc] : 0.f;
    }
    // The loads of chunk c - 1 are issued once chunk c's inputs are in LDS and
    // land while chunk c computes.
    Rows<D, TI> rk, rq;
    Rows<BV, TO> ro;
    CCm nm, pm;
    double gv = 0.0;
    float bv = 0.f;
    auto fetch = [&](int c) {
        const int t0 = c * BC, n = min(BC, L - t0);
        const size_t row0 = ((size_t)b * L + t0) * H + h;
        const float *gc = gnp + (unit * NC + c) * GNP_FLOATS;
        rk.fetch(k + row0 * D, tok, n);
        rq.fetch(q + row0 * D, tok, n);
        ro.fetch(dout + row0 * D + vb * BV, tok, n);
        nm.fetch(gc + G_FLOATS);
        pm.fetch(gc + G_FLOATS + BC * BC);
        if (threadIdx.x < BC) {
            gv = reinterpret_cast<const double *>(gc)[threadIdx.x];
            bv = threadIdx.x < n ? beta[row0 + (size_t)threadIdx.x * H] : 0.f;
        }
    };
    fetch(NC - 1);
    for (int c = NC - 1; c >= 0; --c) {
        const int t0 = c * BC, n = min(BC, L - t0);
        __syncthreads();
        float *dso = dsws + (unit * NC + c) * (size_t)D * D;
        for (int idx = threadIdx.x; idx < D * BV; idx += BNT) {
            const int r = idx / BV, cc = idx % BV;
            dso[r * D + vb * BV + cc] = dS[r * VP + cc];
        }
        rk.put(Ks, DP);
        rq.put(Qs, DP);
        ro.put(dOs, VP);
        nm.put(Ns);
        pm.put(Ps);
        if (threadIdx.x < BC) {
            g[threadIdx.x] = gv;
            bt[threadIdx.x] = bv;
        }
        if (c > 0) fetch(c - 1);
        __syncthreads();
        const double gC = g[n - 1];
        {   // dU = P^T dO + diag(gamma_C / gamma) K dS'
            // two partial sums per tile and product (even, odd k-steps)
            f32x4 a1[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, a2[2] = {a1[0], a1[0]};
            f32x4 b1[2] = {a1[0], a1[0]}, b2[2] = {a1[0], a1[0]};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 8) {
                const float pa = Ps[(k0 + lq) * CPp + ra], pb = Ps[(k0 + 4 + lq) * CPp + ra];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    a1[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, dOs[(k0 + lq) * VP + 16 * j + lr], a1[j], 0, 0, 0);
                    b1[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(pb, dOs[(k0 + 4 + lq) * VP + 16 * j + lr], b1[j], 0, 0, 0);
                }
            }
#pragma unroll 4
            for (int k0 = 0; k0 < D; k0 += 8) {
                const float ka = Ks[ra * DP + k0 + lq], kb = Ks[ra * DP + k0 + 4 + lq];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    a2[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, dS[(k0 + lq) * VP + 16 * j + lr], a2[j], 0, 0, 0);
                    b2[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(kb, dS[(k0 + 4 + lq) * VP + 16 * j + lr], b2[j], 0, 0, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                a1[j] += b1[j];
                a2[j] += b2[j];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = R0 + 4 * lq + r;
                    dUs[t * VP + 16 * j + lr] = fmaf(dexp2(gC, g[t]), a2[j][r], a1[j][r]);
                }
        }
        __syncthreads();
        {   // dR = diag(beta) N^T dU, kept as diag(gamma) dR for the state update
            f32x4 p[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 4) {   // two partial sums per tile
                const int h2 = (k0 >> 2) & 1;
                const float na = Ns[(k0 + lq) * CPp + ra];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    p[h2][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(na, dUs[(k0 + lq) * VP + 16 * j + lr], p[h2][j], 0, 0, 0);
            }
            const f32x4 a[2] = {p[0][0] + p[1][0], p[0][1] + p[1][1]};
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = R0 + 4 * lq + r, o = t * VP + 16 * j + lr;
                    dRs[o] = dexp2(g[t], 0.0) * bt[t] * a[j][r];
                    dOs[o] *= dexp2(g[t], 0.0);   // diag(gamma) dO
                }
        }
        __syncthreads();
        {   // dS = Q^T diag(gamma) dO + gamma_C dS' - K^T diag(gamma) dR  (wave w: state rows SR0 ..)
            f32x4 a[NR][2];
#pragma unroll
            for (int x = 0; x < NR; ++x) a[x][0] = a[x][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k0 = 0; k0 < BC; k0 += 4) {
                const int kk = k0 + lq;
                const float o0 = dOs[kk * VP + lr], o1 = dOs[kk * VP + 16 + lr];
                const float r0 = -dRs[kk * VP + lr], r1 = -dRs[kk * VP + 16 + lr];
#pragma unroll
                for (int x = 0; x < NR; ++x) {
                    const float qt = Qs[kk * DP + SR0 + 16 * x + lr], kt = Ks[kk * DP + SR0 + 16 * x + lr];
                    a[x][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(qt, o0, a[x][0], 0, 0, 0);
                    a[x][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(qt, o1, a[x][1], 0, 0, 0);
                    a[x][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt, r0, a[x][0], 0, 0, 0);
                    a[x][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt, r1, a[x][1], 0, 0, 0);
                }
            }
            const float gam = dexp2(gC, 0.0);
#pragma unroll
            for (int x = 0; x < NR; ++x)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float &y = dS[(SR0 + 16 * x + 4 * lq + r) * VP + 16 * j + lr];
                        y = fmaf(gam, y, a[x][j][r]);
                    }
        }
    }
    __syncthreads();
    if (dstate_in)
        for (int idx = threadIdx.x; idx < D * BV; idx += BNT) {
            const int r = idx / BV, cc = idx % BV;
            dstate_in[(unit * D + r) * D + vb * BV + cc] = dS[r * VP + cc];
        }
}

// ---------------------------------------------------------------------------
// Per-chunk gradients.  The value dimension is walked in blocks of 16 columns;
// dQ, dK (C x D) and dP, dTm (C x C) accumulate in registers across blocks.
// Every product runs on the fp32 matrix cores (v_mfma_f32_16x16x4f32: exact
// fp32 products, fp32 sums), one 16 x 16 output tile per instruction chain.
// Wave w owns rows 16w .. 16w + 15 (tokens) of every row-partitioned product;
// in a tile, lane l holds rows 4 (l / 16) + r, r < 4, of column l % 16, and
// reads A(row l % 16, k = l / 16) and B(k = l / 16, column l % 16) per k-step.
template <int D, typename TI, typename TO>
__global__ __launch_bounds__(BNT) void bwd_grads_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                        const TI *__restrict__ v, const TO *__restrict__ dout,
                                                        const float *__restrict__ beta,
                                                        const float *__restrict__ gnp,
                                                        const float *__restrict__ sws,
                                                        const float *__restrict__ dsws, float *__restrict__ dq,
                                                        float *__restrict__ dk, float *__restrict__ dv,
                                                        float *__restrict__ dlog_alpha, float *__restrict__ dbeta,
                                                        int L, int H, int NC) {
    // Row pitches are multiples of four floats: where a product's operand row is
    // contiguous in k, a lane reads its four k values with one 16-byte load (in
    // a 16-wide k block, product m takes k = 4 (l / 16) + m from lane l, which
    // covers each k once), and the K, Q rows and the 16-column value blocks are
    // read that way.
    constexpr int BV = 16, DP = D + 4, VP = BV + 4;
    constexpr int NJ = D / 16, NP = BC / 16;   // 16-column tiles of dQ/dK and of dP/dTm
    static_assert(BNT == 256 && BC == 64, "four waves of 16 token rows");
    // phase-1 buffers (per value block) and phase-2 buffers (C x C) share one region
    constexpr int P1 = 2 * D * VP + 6 * BC * VP;
    constexpr int P2 = 3 * BC * CPp;
    constexpr int UN = P1 > P2 ? P1 : P2;
    __shared__ __attribute__((aligned(16))) float Qs[BC * DP], Ks[BC * DP], un[UN];
    __shared__ float Ns[BC * CPp], Ps[BC * CPp];
    __shared__ float bt[BC], gq[BC], gk[BC], gd[BC], red[BNT];
    __shared__ double g[BC];
    float *Sb = un, *dSb = Sb + D * VP, *Vb = dSb + D * VP, *dOb = Vb + BC * VP, *Rb = dOb + BC * VP,
          *Ub = Rb + BC * VP, *dUb = Ub + BC * VP, *dRb = dUb + BC * VP;
    float *X1 = un, *X2 = un + BC * CPp, *X3 = un + 2 * BC * CPp;

    const int c = blockIdx.x % NC;
    const size_t unit = blockIdx.x / NC;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const int t0 = c * BC, n = min(BC, L - t0);
    const size_t tok = (size_t)H * D;
    const size_t row0 = ((size_t)b * L + t0) * H + h;
    const float *gc = gnp + (unit * NC + c) * GNP_FLOATS;
    const float *Sc = sws + (unit * NC + c) * (size_t)D * D;
    const float *dSc = dsws + (unit * NC + c) * (size_t)D * D;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int R0 = 16 * __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ra = R0 + lr;   // this lane's A-operand row

    {
        Rows<D, TI> rk, rq;
        CCm nm, pm;
        rk.fetch(k + row0 * D, tok, n);
        rq.fetch(q + row0 * D, tok, n);
        nm.fetch(gc + G_FLOATS);
        pm.fetch(gc + G_FLOATS + BC * BC);
        rk.put(Ks, DP);
        rq.put(Qs, DP);
        nm.put(Ns);
        pm.put(Ps);
    }
    if (tid < BC) {
        g[tid] = reinterpret_cast<const double *>(gc)[tid];
        bt[tid] = tid < n ? beta[row0 + (size_t)tid * H] : 0.f;
    }
    float sdot = 0.f;
    f32x4 aq[NJ], ak[NJ], ap[NP], at[NP];
#pragma unroll
    for (int j = 0; j < NJ; ++j) aq[j] = ak[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NP; ++j) ap[j] = at[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    const double gC = g[n - 1];
    const float ea = dexp2(g[ra], 0.0), eca = dexp2(gC, g[ra]);   // gamma, gamma_C / gamma of row ra
    // gate row terms of this lane's accumulator rows t = R0 + 4 (lane / 16) + r,
    // summed over the value blocks: gamma <dO, QS>, -gamma <dR, KS>, (gamma_C/gamma) <U, KdS>
    float gqr[4] = {0.f, 0.f, 0.f, 0.f}, gkr[4] = {0.f, 0.f, 0.f, 0.f}, gdr[4] = {0.f, 0.f, 0.f, 0.f};

    // A value block's S and dS' columns (16-byte pieces), V and dO columns: the
    // loads of block vb + 1 are issued once block vb is in LDS and land while it
    // computes.
    constexpr int SP = D * BV / 4 / BNT;   // 16-byte pieces of S per thread
    u32x4 xs[SP], xd[SP];
    Rows<BV, TI> rv;
    Rows<BV, TO> ro;
    auto fetch = [&](int vb) {
#pragma unroll
        for (int i = 0; i < SP; ++i) {
            const int e = 4 * (tid + BNT * i), r = e / BV, cc = e % BV;
            xs[i] = *reinterpret_cast<const u32x4 *>(Sc + r * D + vb * BV + cc);
            xd[i] = *reinterpret_cast<const u32x4 *>(dSc + r * D + vb * BV + cc);
        }
        rv.fetch(v + row0 * D + vb * BV, tok, n);
        ro.fetch(dout + row0 * D + vb * BV, tok, n);
    };
    fetch(0);
    for (int vb = 0; vb < D / BV; ++vb) {
#pragma unroll
        for (int i = 0; i < SP; ++i) {
            const int e = 4 * (tid + BNT * i), r = e / BV, cc = e % BV;
            const f32x4 a = {__uint_as_float(xs[i][0]), __uint_as_float(xs[i][1]), __uint_as_float(xs[i][2]),
                             __uint_as_float(xs[i][3])};
            const f32x4 d2 = {__uint_as_float(xd[i][0]), __uint_as_float(xd[i][1]), __uint_as_float(xd[i][2]),
                              __uint_as_float(xd[i][3])};
            *reinterpret_cast<f32x4 *>(&Sb[r * VP + cc]) = a;
            *reinterpret_cast<f32x4 *>(&dSb[r * VP + cc]) = d2;
#pragma unroll
            for (int j = 0; j < 4; ++j) sdot = fmaf(a[j], d2[j], sdot);
        }
        rv.put(Vb, VP);
        ro.put(dOb, VP);
        if (vb + 1 < D / BV) fetch(vb + 1);
        __syncthreads();
        // KS = K S, QS = Q S, KdS = K dS' (C x BV), kept in registers;  R = V - diag(gamma) KS
        f32x4 ks = {0.f, 0.f, 0.f, 0.f}, qs = ks, kds = ks;
#pragma unroll 2
        for (int kb = 0; kb < D; kb += 16) {
            const f32x4 ka = *reinterpret_cast<const f32x4 *>(&Ks[ra * DP + kb + 4 * lq]);
            const f32x4 qa = *reinterpret_cast<const f32x4 *>(&Qs[ra * DP + kb + 4 * lq]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int kk = kb + 4 * lq + m;
                const float sb = Sb[kk * VP + lr], dsb = dSb[kk * VP + lr];
                ks = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[m], sb, ks, 0, 0, 0);
                qs = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[m], sb, qs, 0, 0, 0);
                kds = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[m], dsb, kds, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = (R0 + 4 * lq + r) * VP + lr;
            Rb[o] = Vb[o] - dexp2(g[R0 + 4 * lq + r], 0.0) * ks[r];
        }
        __syncthreads();
        f32x4 u4;   // U, this lane's accumulator rows
        {   // U = N diag(beta) R ; dU = P^T dO + diag(gamma_C/gamma) K dS'
            // four partial sums per product (k-step mod 4): eight independent chains
            f32x4 p1[4], p2[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) p1[x] = p2[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 4) {
                const int kk = k0 + lq, h4 = (k0 >> 2) & 3;
                p1[h4] = __builtin_amdgcn_mfma_f32_16x16x4f32(Ns[ra * CPp + kk], bt[kk] * Rb[kk * VP + lr], p1[h4], 0, 0, 0);
                p2[h4] = __builtin_amdgcn_mfma_f32_16x16x4f32(Ps[kk * CPp + ra], dOb[kk * VP + lr], p2[h4], 0, 0, 0);
            }
            u4 = (p1[0] + p1[1]) + (p1[2] + p1[3]);
            const f32x4 a2 = (p2[0] + p2[1]) + (p2[2] + p2[3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = R0 + 4 * lq + r, o = t * VP + lr;
                Ub[o] = u4[r];
                dUb[o] = fmaf(dexp2(gC, g[t]), kds[r], a2[r]);
            }
        }
        __syncthreads();
        {   // dR = diag(beta) N^T dU  (= dV)
            f32x4 p1[4];   // four partial sums (k-step mod 4)
#pragma unroll
            for (int x = 0; x < 4; ++x) p1[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 4) {
                const int kk = k0 + lq, h4 = (k0 >> 2) & 3;
                p1[h4] = __builtin_amdgcn_mfma_f32_16x16x4f32(Ns[kk * CPp + ra], dUb[kk * VP + lr], p1[h4], 0, 0, 0);
            }
            const f32x4 a1 = (p1[0] + p1[1]) + (p1[2] + p1[3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = R0 + 4 * lq + r;
                const float x = bt[t] * a1[r];
                dRb[t * VP + lr] = x;
                if (t < n) dv[(row0 + (size_t)t * H) * D + vb * BV + lr] = x;
                // gate row terms: this block's 16 columns of row t sit in the 16
                // lanes of this lane's group; reduce across them
                float x1 = dOb[t * VP + lr] * qs[r], x2 = x * ks[r], x3 = u4[r] * kds[r];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    x1 += __shfl_xor(x1, o);
                    x2 += __shfl_xor(x2, o);
                    x3 += __shfl_xor(x3, o);
                }
                const float e = dexp2(g[t], 0.0);
                gqr[r] += e * x1;
                gkr[r] -= e * x2;
                gdr[r] += dexp2(gC, g[t]) * x3;
            }
        }
        __syncthreads();
        // register accumulations over this value block (k = value column s)
        //   dQ += diag(gamma) dO S^T ; dK += diag(gamma_C/gamma) U dS'^T - diag(gamma) dR S^T
        //   dP += dO U^T ; dTm += dU R^T
        {   // value column s = 4 (lane / 16) + m in product m
            const f32x4 o4 = *reinterpret_cast<const f32x4 *>(&dOb[ra * VP + 4 * lq]);
            const f32x4 du4 = *reinterpret_cast<const f32x4 *>(&dUb[ra * VP + 4 * lq]);
            const f32x4 ua4 = *reinterpret_cast<const f32x4 *>(&Ub[ra * VP + 4 * lq]);
            const f32x4 ra4 = *reinterpret_cast<const f32x4 *>(&dRb[ra * VP + 4 * lq]);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const f32x4 sq = *reinterpret_cast<const f32x4 *>(&Sb[(16 * j + lr) * VP + 4 * lq]);
                const f32x4 sd = *reinterpret_cast<const f32x4 *>(&dSb[(16 * j + lr) * VP + 4 * lq]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    aq[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ea * o4[m], sq[m], aq[j], 0, 0, 0);
                    ak[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(eca * ua4[m], sd[m], ak[j], 0, 0, 0);
                    ak[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(-ea * ra4[m], sq[m], ak[j], 0, 0, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const f32x4 ub = *reinterpret_cast<const f32x4 *>(&Ub[(16 * j + lr) * VP + 4 * lq]);
                const f32x4 rb = *reinterpret_cast<const f32x4 *>(&Rb[(16 * j + lr) * VP + 4 * lq]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    ap[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(o4[m], ub[m], ap[j], 0, 0, 0);
                    at[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(du4[m], rb[m], at[j], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // ---- phase 2: C x C algebra (buffers X1..X3 replace the value-block buffers) ----
    // (a) X1 = dP o Gam (lower incl, rows < n), X2 = dTm, X3 = Q K^T
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        f32x4 qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int kb = 0; kb < D; kb += 16) {
            const f32x4 qa = *reinterpret_cast<const f32x4 *>(&Qs[ra * DP + kb + 4 * lq]);
            const f32x4 kb4 = *reinterpret_cast<const f32x4 *>(&Ks[(16 * j + lr) * DP + kb + 4 * lq]);
#pragma unroll
            for (int m = 0; m < 4; ++m) qk = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[m], kb4[m], qk, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = R0 + 4 * lq + r, s = 16 * j + lr;
            const float gam = dexp2(g[t], g[min(s, t)]);
            X1[t * CPp + s] = (s <= t && t < n) ? ap[j][r] * gam : 0.f;
            X2[t * CPp + s] = at[j][r];
            X3[t * CPp + s] = qk[r];
        }
    }
    __syncthreads();
    // (b) dQ += (dP o Gam) K ; dK += (dP o Gam)^T Q ; X = dP o P = X1 o QK^T into Ps
    //     (P is no longer needed) ; dbeta from Tm = N diag(beta): sum_s dTm_st N_st
#pragma unroll 4
    for (int k0 = 0; k0 < BC; k0 += 4) {
        const int kk = k0 + lq;
        const float x = X1[ra * CPp + kk], xt = X1[kk * CPp + ra];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            aq[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, Ks[kk * DP + 16 * j + lr], aq[j], 0, 0, 0);
            ak[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xt, Qs[kk * DP + 16 * j + lr], ak[j], 0, 0, 0);
        }
    }
    for (int idx = tid; idx < BC * BC; idx += BNT) {
        const int t = idx / BC, s = idx % BC;
        Ps[t * CPp + s] = X1[t * CPp + s] * X3[t * CPp + s];
    }
    float dbt = 0.f;
    if (tid < BC) {
        const int t = tid;
        for (int s = 0; s < BC; ++s) dbt = fmaf(X2[s * CPp + t], Ns[s * CPp + t], dbt);
    }
    __syncthreads();
    // (c) T1 = N^T dTm diag(beta) into X1 ; X3 = K K^T
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f}, kk4 = a;
#pragma unroll 4
        for (int k0 = 0; k0 < BC; k0 += 4)
            a = __builtin_amdgcn_mfma_f32_16x16x4f32(Ns[(k0 + lq) * CPp + ra], X2[(k0 + lq) * CPp + 16 * j + lr], a,
                                                    0, 0, 0);
#pragma unroll 4
        for (int kb = 0; kb < D; kb += 16) {
            const f32x4 ka = *reinterpret_cast<const f32x4 *>(&Ks[ra * DP + kb + 4 * lq]);
            const f32x4 kb4 = *reinterpret_cast<const f32x4 *>(&Ks[(16 * j + lr) * DP + kb + 4 * lq]);
#pragma unroll
            for (int m = 0; m < 4; ++m) kk4 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[m], kb4[m], kk4, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = R0 + 4 * lq + r, s = 16 * j + lr;
            X1[t * CPp + s] = a[r] * bt[s];
            X3[t * CPp + s] = kk4[r];
        }
    }
    __syncthreads();
    // (d) dA = -T1 N^T, strict lower part, into X2
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k0 = 0; k0 < BC; k0 += 4)
            a = __builtin_amdgcn_mfma_f32_16x16x4f32(X1[ra * CPp + k0 + lq], Ns[(16 * j + lr) * CPp + k0 + lq], a, 0,
                                                    0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = R0 + 4 * lq + r, s = 16 * j + lr;
            X2[t * CPp + s] = s < t ? -a[r] : 0.f;
        }
    }
    __syncthreads();
    // (e) E = dA beta_t Gam into X1 ; X += dA o A (A = beta_t K K^T Gam) ;
    //     dbeta from A: sum_s dA_ts (k_t . k_s) Gam_ts
    for (int idx = tid; idx < BC * BC; idx += BNT) {
        const int t = idx / BC, s = idx % BC;
        const float gts = s < t ? dexp2(g[t], g[s]) : 0.f;
        const float kg = X3[t * CPp + s] * gts;
        X1[t * CPp + s] = X2[t * CPp + s] * bt[t] * gts;
        Ps[t * CPp + s] = fmaf(X2[t * CPp + s], bt[t] * kg, Ps[t * CPp + s]);
    }
    if (tid < BC) {
        const int t = tid;
        for (int s = 0; s < t; ++s) dbt = fmaf(X2[t * CPp + s], X3[t * CPp + s] * dexp2(g[t], g[s]), dbt);
    }
    __syncthreads();
    // (f) dK += E K + E^T K
#pragma unroll 4
    for (int k0 = 0; k0 < BC; k0 += 4) {
        const int kk = k0 + lq;
        const float x = X1[ra * CPp + kk], xt = X1[kk * CPp + ra];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float kb = Ks[kk * DP + 16 * j + lr];
            ak[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, kb, ak[j], 0, 0, 0);
            ak[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xt, kb, ak[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = R0 + 4 * lq + r;
        if (t < n)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                dq[(row0 + (size_t)t * H) * D + 16 * j + lr] = aq[j][r];
                dk[(row0 + (size_t)t * H) * D + 16 * j + lr] = ak[j][r];
            }
    }
    if (lr == 0) {   // each accumulator row belongs to one lane group
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            gq[R0 + 4 * lq + r] = gqr[r];
            gk[R0 + 4 * lq + r] = gkr[r];
            gd[R0 + 4 * lq + r] = gdr[r];
        }
    }
    // gate (wave 0, thread j = token j of the chunk).  The pairs i < j <= t of X
    // (lower triangular, rows >= n zero): column suffix sums over t in place
    // (lane i walks column i), then lane j adds row j over i < j.
    if (tid < BC) {
        float acc = 0.f;
#pragma unroll 8
        for (int t = BC - 1; t >= 0; --t) {
            acc += Ps[t * CPp + tid];
            Ps[t * CPp + tid] = acc;
        }
    }
    red[tid] = sdot;
    __syncthreads();
    if (tid < 64) {
        float x = red[tid] + red[tid + 64] + red[tid + 128] + red[tid + 192];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
        const int j = tid;
        // suffix sums of gq + gk over t >= j, exclusive prefix sums of gd over t < j
        float suf = j < n ? gq[j] + gk[j] : 0.f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float z = __shfl_down(suf, o);
            if (j + o < 64) suf += z;
        }
        float pre = j < n ? gd[j] : 0.f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float z = __shfl_up(pre, o);
            if (j >= o) pre += z;
        }
        pre -= j < n ? gd[j] : 0.f;
        float cross = 0.f;
#pragma unroll 8
        for (int i = 0; i < BC; ++i) cross += i < j ? Ps[j * CPp + i] : 0.f;
        if (j < n) {
            dlog_alpha[row0 + (size_t)j * H] = suf + pre + cross + dexp2(gC, 0.0) * x;
            dbeta[row0 + (size_t)j * H] = dbt;
        }
    }
}

template <int D, typename TI, typename TO>
hipError_t launch_bwd_d(const GdnBwdArgs &a, hipStream_t s) {
    const int NC = (a.L + BC - 1) / BC;
    const BwdLayout w = bwd_layout(a.B, a.L, a.H, D);
    unsigned char *ws = static_cast<unsigned char *>(a.ws);
    float *gnp = reinterpret_cast<float *>(ws + w.gnp);
    float *sws = reinterpret_cast<float *>(ws + w.s);
    float *dsws = reinterpret_cast<float *>(ws + w.ds);
    const TI *q = static_cast<const TI *>(a.q), *k = static_cast<const TI *>(a.k), *v = static_cast<const TI *>(a.v);
    const TO *dout = static_cast<const TO *>(a.dout);
    const unsigned units = (unsigned)((size_t)a.B * a.H);
    hipLaunchKernelGGL((bwd_prep_kernel<D, TI>), dim3(units * NC), dim3(BNT), 0, s, q, k, a.alpha, a.beta, gnp, a.L,
                       a.H, NC);
    hipLaunchKernelGGL((bwd_states_kernel<D, TI>), dim3(units * (D / 32)), dim3(BNT), 0, s, k, v, a.beta,
                       a.state_in, gnp, sws, a.L, a.H, NC);
    hipLaunchKernelGGL((bwd_dstate_kernel<D, TI, TO>), dim3(units * (D / 32)), dim3(BNT), 0, s, q, k, dout, a.beta,
                       a.dstate_out, gnp, dsws, a.dstate_in, a.L, a.H, NC);
    hipLaunchKernelGGL((bwd_grads_kernel<D, TI, TO>), dim3(units * NC), dim3(BNT), 0, s, q, k, v, dout, a.beta, gnp,
                       sws, dsws, a.dq, a.dk, a.dv, a.dlog_alpha, a.dbeta, a.L, a.H, NC);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_dt(const GdnBwdArgs &a, hipStream_t s) {
    if (a.qkv_bf16)
        return a.dout_bf16 ? launch_bwd_d<D, uint16_t, uint16_t>(a, s) : launch_bwd_d<D, uint16_t, float>(a, s);
    return a.dout_bf16 ? launch_bwd_d<D, float, uint16_t>(a, s) : launch_bwd_d<D, float, float>(a, s);
}

}  // namespace

size_t gdn_bwd_ws_bytes(int B, int L, int H, int d) { return bwd_layout(B, L, H, d).total; }

hipError_t launch_gdn_bwd(const GdnBwdArgs &a, hipStream_t s) {
    if (a.B == 0 || a.L == 0) return hipSuccess;
    return a.d == 64 ? launch_bwd_dt<64>(a, s) : launch_bwd_dt<128>(a, s);
}

}  // namespace lt2
