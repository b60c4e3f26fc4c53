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
// Four launches; values are held and summed in fp32 apart from those sums
// (bf16 inputs are widened exactly):
//   bwd_prep_kernel    one workgroup per (b, h, chunk): g, N, P into the workspace
//   bwd_states_kernel  one per (b, h, 32-column block): the state entering every chunk
//   bwd_dstate_kernel  one per (b, h, 32-column block), chunks in reverse: the
//                      cotangent of the state leaving every chunk, and dS_0
//   bwd_grads_kernel   one per (b, h, chunk): dv, dq, dk, dbeta, d(log alpha)
// Products run on the matrix cores from LDS operands.  fp32 inputs: the fp32
// instruction (v_mfma_f32_16x16x4f32: exact fp32 products, fp32 sums).  bf16
// inputs: the bf16 instructions, the inputs as they are and every fp32
// intermediate split into hi + lo bf16 halves (about 16 significant bits per
// operand, fp32 sums; K K^T and Q K^T of the inputs are exact).  In the
// gradients kernel the operands that all waves read (N, P^T, the S and dS'
// blocks) are stored split.  Each wave owns 16-row output tiles.  Every load
// of a chunk is issued before the first of them is used.
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
// (pitch CPp unless given), four 16-byte loads per thread.
struct CCm {
    static constexpr int IT = BC * BC / 4 / BNT;
    u32x4 x[IT];
    __device__ __forceinline__ void fetch(const float *src) {
#pragma unroll
        for (int i = 0; i < IT; ++i) x[i] = reinterpret_cast<const u32x4 *>(src)[threadIdx.x + BNT * i];
    }
    __device__ __forceinline__ void put(float *dst, int pitch = CPp) const {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = 4 * (threadIdx.x + BNT * i), r = e / BC, c = e % BC;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[r * pitch + c + j] = __uint_as_float(x[i][j]);
        }
    }
    // as put and put_t, each value stored as a packed hi/lo word (pack_hilo4)
    __device__ __forceinline__ void put_packed(float *dst, int pitch) const;
    __device__ __forceinline__ void put_t_packed(float *dst, int pitch) const;
    // transposed: dst[c * pitch + r] = M[r][c]
    __device__ __forceinline__ void put_t(float *dst, int pitch) const {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = 4 * (threadIdx.x + BNT * i), r = e / BC, c = e % BC;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[(c + j) * pitch + r] = __uint_as_float(x[i][j]);
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
// Sum over each 16-lane row of the wave (lanes 16 i .. 16 i + 15), result in
// every lane of the row: rotations by 8 and 4 within the row, then swaps of
// lane pairs 2 apart and 1 apart within each quad (all DPP moves).
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));   // row_ror:8
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));   // row_ror:4
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));    // quad_perm 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));    // quad_perm 1,0,3,2
    return x;
}

// ---------------------------------------------------------------------------
// g, N = (I + A)^-1 and P of one chunk.  K K^T and Q K^T run on the matrix
// cores in 32-wide k blocks (bf16 inputs: one bf16 instruction per block, whose
// products are exact, with fp32 sums; fp32 inputs: eight fp32 instructions).
// In a block, lane l reads eight consecutive k values 32 kb + 8 (l / 16) ..
// of row l % 16 of both operands.  The inverse takes its 16 x 16 diagonal
// blocks by forward substitution in registers and the blocks below them by
// block distance on the fp32 matrix cores:
//   N_IJ = -N_II sum_{K=J}^{I-1} A_IK N_KJ   (I > J).
template <typename TI>
__device__ __forceinline__ f32x4 gram_block(f32x4 acc, const TI *a, const TI *b);
template <>
__device__ __forceinline__ f32x4 gram_block<uint16_t>(f32x4 acc, const uint16_t *a, const uint16_t *b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8 *>(a),
                                                   *reinterpret_cast<const bf16x8 *>(b), acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 gram_block<float>(f32x4 acc, const float *a, const float *b) {
    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(a), a1 = *reinterpret_cast<const f32x4 *>(a + 4);
    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(b), b1 = *reinterpret_cast<const f32x4 *>(b + 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[s], b0[s], acc, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[s], b1[s], acc, 0, 0, 0);
    return acc;
}
// (I, J) of lower tile number tl (row-major over I >= J)
__device__ __forceinline__ void lower_tile(int tl, int &I, int &J) {
    I = 0;
    while ((I + 1) * (I + 2) / 2 <= tl) ++I;
    J = tl - I * (I + 1) / 2;
}

template <int D, typename TI>
__global__ __launch_bounds__(BNT) void bwd_prep_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                       const float *__restrict__ alpha,
                                                       const float *__restrict__ beta, float *__restrict__ gnp,
                                                       int L, int H, int NC) {
    constexpr int KP = D + 16 / (int)sizeof(TI);   // row pitch (elements): rows stay 16-byte aligned
    constexpr int CQ = BC + 4, NT = BC / 16, NLT = NT * (NT + 1) / 2, MP = (NLT + 3) / 4;
    constexpr int VE = 16 / (int)sizeof(TI), PPR = D / VE, PCS = BC * PPR / BNT;   // 16-byte pieces
    static_assert(BC * PPR % BNT == 0 && 2 * BC * KP * (int)sizeof(TI) >= BC * CQ * 4, "layout");
    __shared__ __attribute__((aligned(16))) TI KQ[2 * BC * KP];   // K, Q; then P
    __shared__ __attribute__((aligned(16))) float As[BC * CQ], Ns[BC * CQ];
    __shared__ float Xs[NT][16 * 17], bt[BC];
    __shared__ double g[BC];
    TI *Ks = KQ, *Qs = KQ + BC * KP;
    float *Ps = reinterpret_cast<float *>(KQ);
    const int c = blockIdx.x % NC;
    const size_t unit = blockIdx.x / NC;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const int t0 = c * BC, n = min(BC, L - t0);
    const size_t row0 = ((size_t)b * L + t0) * H + h;   // (b, t0, h) in [B, L, H]
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    {
        u32x4 kr[PCS], qr[PCS];
#pragma unroll
        for (int i = 0; i < PCS; ++i) {
            const int idx = tid + BNT * i, r = idx / PPR, cc = VE * (idx % PPR);
            const size_t o = (row0 + (size_t)min(r, n - 1) * H) * D + cc;
            kr[i] = *reinterpret_cast<const u32x4 *>(k + o);
            qr[i] = *reinterpret_cast<const u32x4 *>(q + o);
        }
#pragma unroll
        for (int i = 0; i < PCS; ++i) {
            const int idx = tid + BNT * i, r = idx / PPR, cc = VE * (idx % PPR);
            const u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(Ks + r * KP + cc) = r < n ? kr[i] : z;
            *reinterpret_cast<u32x4 *>(Qs + r * KP + cc) = r < n ? qr[i] : z;
        }
    }
    gate_prefix(g, alpha + row0, H, n);
    if (tid < BC) bt[tid] = tid < n ? beta[row0 + (size_t)tid * H] : 0.f;
    // N starts as zero (its blocks above the diagonal stay zero)
    for (int idx = tid; idx < BC * BC; idx += BNT) Ns[(idx / BC) * CQ + idx % BC] = 0.f;
    __syncthreads();
    // A = strict_lower(beta_t Gam_ts k_t . k_s): the lower tiles of K K^T (wave w
    // takes tiles w, w + 4, ...); tiles above the diagonal are never read
    for (int tl = wave; tl < NLT; tl += 4) {
        int I, J;
        lower_tile(tl, I, J);
        const TI *ar = Ks + (16 * I + lr) * KP + 8 * lq, *br = Ks + (16 * J + lr) * KP + 8 * lq;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) acc = gram_block<TI>(acc, ar + 32 * kb, br + 32 * kb);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + 4 * lq + r, s = 16 * J + lr;
            // computed for every element, then selected (see materialize)
            const float v = materialize(bt[t] * dexp2(g[t], g[s]) * acc[r]);
            As[t * CQ + s] = s < t ? v : 0.f;
        }
    }
    // the lower tiles of Q K^T stay in registers until K and Q are dead
    f32x4 pacc[MP];
#pragma unroll
    for (int m = 0; m < MP; ++m) {
        pacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tl = wave + 4 * m;
        if (tl >= NLT) continue;
        int I, J;
        lower_tile(tl, I, J);
        const TI *ar = Qs + (16 * I + lr) * KP + 8 * lq, *br = Ks + (16 * J + lr) * KP + 8 * lq;
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) pacc[m] = gram_block<TI>(pacc[m], ar + 32 * kb, br + 32 * kb);
    }
    __syncthreads();
    // diagonal blocks: wave w solves block w, lane j < 16 its column j
    if (wave < NT && lane < 16) {
        const int o = 16 * wave;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float y = t == lane ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < t; ++s2) y = fmaf(-As[(o + t) * CQ + o + s2], x[s2], y);
            x[t] = y;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) Ns[(o + t) * CQ + o + lane] = x[t];
    }
    __syncthreads();
    // blocks below the diagonal, one block distance at a time (wave w: J = w)
    for (int dist = 1; dist < NT; ++dist) {
        if (wave < NT - dist) {
            const int J = wave, I = wave + dist;
            f32x4 w4 = {0.f, 0.f, 0.f, 0.f};   // W = sum_K A_IK N_KJ
            for (int kb = 16 * J; kb < 16 * I; kb += 4)
                w4 = __builtin_amdgcn_mfma_f32_16x16x4f32(As[(16 * I + lr) * CQ + kb + lq],
                                                         Ns[(kb + lq) * CQ + 16 * J + lr], w4, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) Xs[wave][(4 * lq + r) * 17 + lr] = w4[r];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x4 y = {0.f, 0.f, 0.f, 0.f};   // N_II W
#pragma unroll
            for (int k4 = 0; k4 < 16; k4 += 4)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(Ns[(16 * I + lr) * CQ + 16 * I + k4 + lq],
                                                        Xs[wave][(k4 + lq) * 17 + lr], y, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) Ns[(16 * I + 4 * lq + r) * CQ + 16 * J + lr] = -y[r];
        }
        __syncthreads();
    }
    // P = (Q K^T o Gam) on s <= t, rows < n, into K's space
#pragma unroll
    for (int m = 0; m < MP; ++m) {
        const int tl = wave + 4 * m;
        if (tl >= NLT) continue;
        int I, J;
        lower_tile(tl, I, J);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + 4 * lq + r, s = 16 * J + lr;
            const float v = materialize(dexp2(g[t], g[s]) * pacc[m][r]);
            Ps[t * CQ + s] = (s <= t && t < n) ? v : 0.f;
        }
    }
    __syncthreads();
    float *out = gnp + (unit * NC + c) * GNP_FLOATS;
    if (tid < BC) reinterpret_cast<double *>(out)[tid] = g[tid];
    for (int idx = tid; idx < BC * BC / 4; idx += BNT) {
        const int t = idx / (BC / 4), s = 4 * (idx % (BC / 4));
        f32x4 nv = *reinterpret_cast<const f32x4 *>(&Ns[t * CQ + s]);
        f32x4 pv = *reinterpret_cast<const f32x4 *>(&Ps[t * CQ + s]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (s + e > t) pv[e] = 0.f;   // tiles above the diagonal hold K, Q bytes
        *reinterpret_cast<f32x4 *>(out + G_FLOATS + t * BC + s) = nv;
        *reinterpret_cast<f32x4 *>(out + G_FLOATS + BC * BC + t * BC + s) = pv;
    }
}

// ---------------------------------------------------------------------------
// Matrix-core helpers of the chunk-state and gradients kernels.  A contraction
// runs in 16-wide k blocks: in product m of a block, lane l reads A(row l % 16,
// k = k0 + 4 (l / 16) + m) and B(k = k0 + 4 (l / 16) + m, column l % 16).
// krow4 reads the four k values of a row that is contiguous in k (one 16-byte
// read), kcol4 those of a column (rows 4 apart: with a row pitch of 4 (mod 16)
// words the four lane groups fall on disjoint banks).
__device__ __forceinline__ f32x4 krow4(const float *m, int pitch, int r, int k0, int lq) {
    return *reinterpret_cast<const f32x4 *>(&m[r * pitch + k0 + 4 * lq]);
}
__device__ __forceinline__ f32x4 kcol4(const float *m, int pitch, int col, int k0, int lq) {
    const float *p = &m[(k0 + 4 * lq) * pitch + col];
    return f32x4{p[0], p[pitch], p[2 * pitch], p[3 * pitch]};
}
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}
// The operands of one 16-wide k block in the precision of the inputs.  fp32
// inputs: the four fp32 values feed four v_mfma_f32_16x16x4f32 (exact
// products).  bf16 inputs: v_mfma_f32_16x16x16_bf16 takes the same four k
// values per lane as bf16.  Values known to be bf16 (the widened inputs) go in
// as they are (EX); others are split into hi = bf16(x) and lo = bf16(x - hi),
// and a product sums hi*hi + lo*hi + hi*lo (about 16 significant bits of each
// operand; fp32 sums).
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// bf16(a) in the low half, bf16(b) in the high half (round to nearest even)
__device__ __forceinline__ unsigned bf16_pair(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
template <bool BF, bool EX>
struct Op4 {
    f32x4 f;
};
template <>
struct Op4<true, true> {
    s16x4 hi;
};
template <>
struct Op4<true, false> {
    s16x4 hi, lo;
};
template <bool BF, bool EX>
__device__ __forceinline__ Op4<BF, EX> op4(f32x4 x) {
    Op4<BF, EX> o;
    if constexpr (!BF) {
        o.f = x;
    } else if constexpr (EX) {   // the high halves are the bf16 values
        const u32x2 h = {__builtin_amdgcn_perm(__float_as_uint(x[1]), __float_as_uint(x[0]), 0x07060302u),
                         __builtin_amdgcn_perm(__float_as_uint(x[3]), __float_as_uint(x[2]), 0x07060302u)};
        o.hi = __builtin_bit_cast(s16x4, h);
    } else {
        const unsigned h0 = bf16_pair(x[0], x[1]), h1 = bf16_pair(x[2], x[3]);
        const unsigned l0 = bf16_pair(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xFFFF0000u));
        const unsigned l1 = bf16_pair(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xFFFF0000u));
        o.hi = __builtin_bit_cast(s16x4, u32x2{h0, h1});
        o.lo = __builtin_bit_cast(s16x4, u32x2{l0, l1});
    }
    return o;
}
// Operands that several waves read are split once, where they are written to
// LDS, into one 32-bit word per value: hi in the low half, lo in the high half.
__device__ __forceinline__ f32x4 pack_hilo4(f32x4 x) {
    const unsigned h0 = bf16_pair(x[0], x[1]), h1 = bf16_pair(x[2], x[3]);
    const unsigned l0 = bf16_pair(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xFFFF0000u));
    const unsigned l1 = bf16_pair(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xFFFF0000u));
    return f32x4{__uint_as_float(__builtin_amdgcn_perm(l0, h0, 0x05040100u)),
                 __uint_as_float(__builtin_amdgcn_perm(l0, h0, 0x07060302u)),
                 __uint_as_float(__builtin_amdgcn_perm(l1, h1, 0x05040100u)),
                 __uint_as_float(__builtin_amdgcn_perm(l1, h1, 0x07060302u))};
}
__device__ __forceinline__ Op4<true, false> op4_packed(f32x4 w) {
    const unsigned w0 = __float_as_uint(w[0]), w1 = __float_as_uint(w[1]), w2 = __float_as_uint(w[2]),
                   w3 = __float_as_uint(w[3]);
    Op4<true, false> o;
    o.hi = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(w1, w0, 0x05040100u),
                                           __builtin_amdgcn_perm(w3, w2, 0x05040100u)});
    o.lo = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(w1, w0, 0x07060302u),
                                           __builtin_amdgcn_perm(w3, w2, 0x07060302u)});
    return o;
}
__device__ __forceinline__ float unpack_hilo(float w) {   // hi + lo
    const unsigned u = __float_as_uint(w);
    return __uint_as_float(u << 16) + __uint_as_float(u & 0xFFFF0000u);
}
__device__ __forceinline__ void CCm::put_packed(float *dst, int pitch) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int e = 4 * (threadIdx.x + BNT * i), r = e / BC, c = e % BC;
        const f32x4 w = pack_hilo4(__builtin_bit_cast(f32x4, x[i]));
        *reinterpret_cast<f32x4 *>(&dst[r * pitch + c]) = w;
    }
}
__device__ __forceinline__ void CCm::put_t_packed(float *dst, int pitch) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int e = 4 * (threadIdx.x + BNT * i), r = e / BC, c = e % BC;
        const f32x4 w = pack_hilo4(__builtin_bit_cast(f32x4, x[i]));
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[(c + j) * pitch + r] = w[j];
    }
}
// an operand block of a stored matrix: packed words (bf16 inputs) or fp32 values
template <bool BF>
__device__ __forceinline__ Op4<BF, false> op4_stored(f32x4 x) {
    if constexpr (BF) return op4_packed(x);
    else return op4<false, false>(x);
}

// acc += (A block) (B block) for one 16-wide k block
template <bool BF, bool AE, bool BE>
__device__ __forceinline__ f32x4 mm4(f32x4 acc, const Op4<BF, AE> &a, const Op4<BF, BE> &b) {
    if constexpr (!BF) {
#pragma unroll
        for (int m = 0; m < 4; ++m) acc = mfma4(a.f[m], b.f[m], acc);
    } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, acc, 0, 0, 0);
        if constexpr (!AE) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, acc, 0, 0, 0);
        if constexpr (!BE) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, acc, 0, 0, 0);
    }
    return acc;
}
// A k loop of NK blocks, software-pipelined over two register buffers:
// ld(buf, i) issues block i's operand loads, mm(buf, i) runs its products.
// Block i + 1's loads are issued before block i's products (the scheduling
// barriers keep the compiler from sinking them to their first use).
template <int NK, class LD, class MM>
__device__ __forceinline__ void kpipe(LD &&ld, MM &&mm) {
    ld(0, 0);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        if (i + 1 < NK) ld((i + 1) & 1, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        mm(i & 1, i);
        __builtin_amdgcn_sched_barrier(0);
    }
}
// D x BV fp32 state block: global (row pitch D, columns c0 ..) <-> LDS (pitch VP)
template <int D, int BV, int VP>
__device__ __forceinline__ void state_to_lds(float *dst, const float *src, int c0) {
    for (int idx = threadIdx.x; idx < D * BV / 4; idx += BNT) {
        const int r = idx / (BV / 4), cc = 4 * (idx % (BV / 4));
        *reinterpret_cast<f32x4 *>(&dst[r * VP + cc]) =
            src ? *reinterpret_cast<const f32x4 *>(&src[(size_t)r * D + c0 + cc]) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}
template <int D, int BV, int VP>
__device__ __forceinline__ void state_from_lds(float *dst, const float *src, int c0) {
    for (int idx = threadIdx.x; idx < D * BV / 4; idx += BNT) {
        const int r = idx / (BV / 4), cc = 4 * (idx % (BV / 4));
        *reinterpret_cast<f32x4 *>(&dst[(size_t)r * D + c0 + cc]) = *reinterpret_cast<const f32x4 *>(&src[r * VP + cc]);
    }
}

// ---------------------------------------------------------------------------
// The state entering every chunk, per 32-column block of the value dimension.
// Row pitches: D + 4 (K), 36 (32-column blocks), C + 4 (N).
template <int D, typename TI>
__global__ __launch_bounds__(BNT) void bwd_states_kernel(const TI *__restrict__ k, const TI *__restrict__ v,
                                                         const float *__restrict__ beta,
                                                         const float *__restrict__ state_in,
                                                         const float *__restrict__ gnp, float *__restrict__ sws,
                                                         int L, int H, int NC) {
    constexpr int BV = 32, DP = D + 4, VP = BV + 4, CQ = BC + 4;
    constexpr int NB = D / BV, KD = D / 16, KC = BC / 16;
    constexpr bool BF = sizeof(TI) == 2;   // bf16 inputs: bf16 matrix cores (K exact, the rest split)
    __shared__ __attribute__((aligned(16))) float Ss[D * VP], Ks[BC * DP], Vs[BC * VP], Ns[BC * CQ], Rs[BC * VP],
        Us[BC * VP];
    __shared__ float bt[BC];
    __shared__ double g[BC];
    // matrix-core roles (16 x 16 output tiles): wave w owns token rows
    // 16w .. 16w + 15 of the C x 32 products and state rows SR0 .. SR0 + 16 NR - 1
    constexpr int NR = D / 64;
    static_assert(BNT == 256 && BC == 64 && BV == 32, "four waves, two 16-column tiles");
    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R0 = 16 * wv, ra = R0 + lr, SR0 = 16 * NR * wv;
    // the NB column blocks of a (b, h) read the same K, N (and Q, P) rows: give
    // them one XCD, so that one L2 serves all of them
    const int bid = xcd_logical(blockIdx.x, gridDim.x);
    const int vb = bid % NB;
    const size_t unit = bid / NB;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const size_t tok = (size_t)H * D;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    state_to_lds<D, BV, VP>(Ss, state_in ? state_in + unit * D * D : nullptr, vb * BV);
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
        rk.put(Ks, DP);
        rv.put(Vs, VP);
        nm.put(Ns, CQ);
        if (threadIdx.x < BC) {
            g[threadIdx.x] = gv;
            bt[threadIdx.x] = bv;
        }
        // the state entering chunk c (stored after the puts: their waits then
        // cover only loads, not these stores)
        state_from_lds<D, BV, VP>(sws + (unit * NC + c) * (size_t)D * D, Ss, vb * BV);
        if (c + 1 < NC) fetch(c + 1);
        __syncthreads();
        const double gC = g[n - 1];
        float er[4], ecr[4], br[4];   // gamma, gamma_C / gamma, beta of rows R0 + 4 (lane / 16) + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = R0 + 4 * lq + r;
            er[r] = dexp2(g[t], 0.0);
            ecr[r] = dexp2(gC, g[t]);
            br[r] = bt[t];
        }
        {   // R' = diag(beta) (V - diag(gamma) K S); two partial sums per tile (even, odd k blocks)
            f32x4 p[2][2] = {{z4, z4}, {z4, z4}}, ka[2], sb[2][2];
            kpipe<KD>(
                [&](int u, int i) {
                    ka[u] = krow4(Ks, DP, ra, 16 * i, lq);
#pragma unroll
                    for (int j = 0; j < 2; ++j) sb[u][j] = kcol4(Ss, VP, 16 * j + lr, 16 * i, lq);
                },
                [&](int u, int i) {
                    const auto a = op4<BF, BF>(ka[u]);
#pragma unroll
                    for (int j = 0; j < 2; ++j) p[i & 1][j] = mm4(p[i & 1][j], a, op4<BF, false>(sb[u][j]));
                });
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = (R0 + 4 * lq + r) * VP + 16 * j + lr;
                    Rs[o] = br[r] * (Vs[o] - er[r] * (p[0][j][r] + p[1][j][r]));
                }
        }
        __syncthreads();
        {   // U' = diag(gamma_C / gamma) N R'
            f32x4 p[2][2] = {{z4, z4}, {z4, z4}}, na[2], rb[2][2];
            kpipe<KC>(
                [&](int u, int i) {
                    na[u] = krow4(Ns, CQ, ra, 16 * i, lq);
#pragma unroll
                    for (int j = 0; j < 2; ++j) rb[u][j] = kcol4(Rs, VP, 16 * j + lr, 16 * i, lq);
                },
                [&](int u, int i) {
                    const auto a = op4<BF, false>(na[u]);
#pragma unroll
                    for (int j = 0; j < 2; ++j) p[i & 1][j] = mm4(p[i & 1][j], a, op4<BF, false>(rb[u][j]));
                });
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Us[(R0 + 4 * lq + r) * VP + 16 * j + lr] = ecr[r] * (p[0][j][r] + p[1][j][r]);
        }
        __syncthreads();
        {   // S = gamma_C S + K^T U'  (wave w: state rows 16 (w NR + x) .., both column tiles)
            f32x4 a[NR][2], kt[2][NR], ub[2][2];
#pragma unroll
            for (int x = 0; x < NR; ++x) a[x][0] = a[x][1] = z4;
            kpipe<KC>(
                [&](int u, int i) {
#pragma unroll
                    for (int x = 0; x < NR; ++x) kt[u][x] = kcol4(Ks, DP, SR0 + 16 * x + lr, 16 * i, lq);
#pragma unroll
                    for (int j = 0; j < 2; ++j) ub[u][j] = kcol4(Us, VP, 16 * j + lr, 16 * i, lq);
                },
                [&](int u, int) {
                    const Op4<BF, false> b0 = op4<BF, false>(ub[u][0]), b1 = op4<BF, false>(ub[u][1]);
#pragma unroll
                    for (int x = 0; x < NR; ++x) {
                        const auto a2 = op4<BF, BF>(kt[u][x]);
                        a[x][0] = mm4(a[x][0], a2, b0);
                        a[x][1] = mm4(a[x][1], a2, b1);
                    }
                });
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
// dS' entering every chunk from the right (the cotangent of the state leaving
// it), per 32-column block, chunks in reverse; the final one is d state_in.
// Pitches as in the chunk-state kernel; P is held transposed (read as P^T).
template <int D, typename TI, typename TO>
__global__ __launch_bounds__(BNT) void bwd_dstate_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                         const TO *__restrict__ dout, const float *__restrict__ beta,
                                                         const float *__restrict__ dstate_out,
                                                         const float *__restrict__ gnp, float *__restrict__ dsws,
                                                         float *__restrict__ dstate_in, int L, int H, int NC) {
    constexpr int BV = 32, DP = D + 4, VP = BV + 4, CQ = BC + 4;
    constexpr int NB = D / BV, KD = D / 16, KC = BC / 16;
    // bf16 inputs: bf16 matrix cores (K, Q exact; dO exact when it is bf16; the rest split)
    constexpr bool BF = sizeof(TI) == 2, OX = BF && sizeof(TO) == 2;
    __shared__ __attribute__((aligned(16))) float dS[D * VP], Ks[BC * DP], Qs[BC * DP], dOs[BC * VP], Ns[BC * CQ],
        Pt[BC * CQ], dUs[BC * VP], dRs[BC * VP];
    __shared__ float bt[BC];
    __shared__ double g[BC];
    // matrix-core roles as in the chunk-state kernel
    constexpr int NR = D / 64;
    static_assert(BNT == 256 && BC == 64 && BV == 32, "four waves, two 16-column tiles");
    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R0 = 16 * wv, ra = R0 + lr, SR0 = 16 * NR * wv;
    // the NB column blocks of a (b, h) read the same K, N (and Q, P) rows: give
    // them one XCD, so that one L2 serves all of them
    const int bid = xcd_logical(blockIdx.x, gridDim.x);
    const int vb = bid % NB;
    const size_t unit = bid / NB;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const size_t tok = (size_t)H * D;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    state_to_lds<D, BV, VP>(dS, dstate_out ? dstate_out + unit * D * D : nullptr, vb * BV);
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
    // L2 prefetch two chunks ahead of the register fetch: one 4-byte load per
    // 128-byte line of chunk c's K and Q rows, N and P (shared by the unit's NB
    // column blocks, so each block touches one NB-th of them) and this block's dO
    // rows, so the fetch a chunk later hits L2.  The word only reaches an empty
    // asm a chunk later, so nothing waits for it in between.
    unsigned pf_word = 0u;
    auto l2_touch = [&](int c) {
        asm volatile("" ::"v"(pf_word));   // the previous touch has landed by now
        if (c < 0) return;
        const int t0 = c * BC, last = min(BC, L - t0) - 1;
        const size_t row0 = ((size_t)b * L + t0) * H + h;
        constexpr int KL = D * (int)sizeof(TI) / 128;       // lines per K (Q) row
        constexpr int NPL = 2 * BC * BC * 4 / 128;          // lines of N and P
        constexpr int SHARED = 2 * BC * KL + NPL;           // lines the NB blocks share
        constexpr int PER = (SHARED + NB - 1) / NB;
        const int i = (int)threadIdx.x;
        const unsigned *p = nullptr;
        if (i < PER) {
            const int line = vb * PER + i;
            if (line < BC * KL) {
                p = reinterpret_cast<const unsigned *>(k + (row0 + (size_t)min(line / KL, last) * H) * D) +
                    (line % KL) * 32;
            } else if (line < 2 * BC * KL) {
                const int j = line - BC * KL;
                p = reinterpret_cast<const unsigned *>(q + (row0 + (size_t)min(j / KL, last) * H) * D) + (j % KL) * 32;
            } else if (line < SHARED) {
                p = reinterpret_cast<const unsigned *>(gnp + (unit * NC + c) * GNP_FLOATS + G_FLOATS) +
                    (line - 2 * BC * KL) * 32;
            }
        } else if (i < PER + BC) {   // this block's dO rows (BV columns, within one line)
            p = reinterpret_cast<const unsigned *>(dout + (row0 + (size_t)min(i - PER, last) * H) * D + vb * BV);
        }
        if (p) pf_word = *p;
    };
    fetch(NC - 1);
    for (int c = NC - 1; c >= 0; --c) {
        const int t0 = c * BC, n = min(BC, L - t0);
        __syncthreads();
        rk.put(Ks, DP);
        rq.put(Qs, DP);
        ro.put(dOs, VP);
        nm.put(Ns, CQ);
        pm.put_t(Pt, CQ);
        if (threadIdx.x < BC) {
            g[threadIdx.x] = gv;
            bt[threadIdx.x] = bv;
        }
        // dS' entering chunk c (stored after the puts, as in the chunk-state kernel)
        state_from_lds<D, BV, VP>(dsws + (unit * NC + c) * (size_t)D * D, dS, vb * BV);
        if (c > 0) fetch(c - 1);
        l2_touch(c - 2);
        __syncthreads();
        const double gC = g[n - 1];
        float er[4], ecr[4], br[4];   // gamma, gamma_C / gamma, beta of rows R0 + 4 (lane / 16) + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = R0 + 4 * lq + r;
            er[r] = dexp2(g[t], 0.0);
            ecr[r] = dexp2(gC, g[t]);
            br[r] = bt[t];
        }
        {   // dU = P^T dO + diag(gamma_C / gamma) K dS'
            f32x4 a1[2][2] = {{z4, z4}, {z4, z4}}, a2[2][2] = {{z4, z4}, {z4, z4}};
            f32x4 pa[2], ob[2][2];
            kpipe<KC>(
                [&](int u, int i) {
                    pa[u] = krow4(Pt, CQ, ra, 16 * i, lq);
#pragma unroll
                    for (int j = 0; j < 2; ++j) ob[u][j] = kcol4(dOs, VP, 16 * j + lr, 16 * i, lq);
                },
                [&](int u, int i) {
                    const auto a = op4<BF, false>(pa[u]);
#pragma unroll
                    for (int j = 0; j < 2; ++j) a1[i & 1][j] = mm4(a1[i & 1][j], a, op4<BF, OX>(ob[u][j]));
                });
            f32x4 ka[2], sb[2][2];
            kpipe<KD>(
                [&](int u, int i) {
                    ka[u] = krow4(Ks, DP, ra, 16 * i, lq);
#pragma unroll
                    for (int j = 0; j < 2; ++j) sb[u][j] = kcol4(dS, VP, 16 * j + lr, 16 * i, lq);
                },
                [&](int u, int i) {
                    const auto a = op4<BF, BF>(ka[u]);
#pragma unroll
                    for (int j = 0; j < 2; ++j) a2[i & 1][j] = mm4(a2[i & 1][j], a, op4<BF, false>(sb[u][j]));
                });
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dUs[(R0 + 4 * lq + r) * VP + 16 * j + lr] =
                        fmaf(ecr[r], a2[0][j][r] + a2[1][j][r], a1[0][j][r] + a1[1][j][r]);
        }
        __syncthreads();
        {   // dR = diag(beta) N^T dU, kept as diag(gamma) dR for the state update
            f32x4 p[2][2] = {{z4, z4}, {z4, z4}}, na[2], ub[2][2];
            kpipe<KC>(
                [&](int u, int i) {
                    na[u] = kcol4(Ns, CQ, ra, 16 * i, lq);
#pragma unroll
                    for (int j = 0; j < 2; ++j) ub[u][j] = kcol4(dUs, VP, 16 * j + lr, 16 * i, lq);
                },
                [&](int u, int i) {
                    const auto a = op4<BF, false>(na[u]);
#pragma unroll
                    for (int j = 0; j < 2; ++j) p[i & 1][j] = mm4(p[i & 1][j], a, op4<BF, false>(ub[u][j]));
                });
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = (R0 + 4 * lq + r) * VP + 16 * j + lr;
                    dRs[o] = er[r] * br[r] * (p[0][j][r] + p[1][j][r]);
                    dOs[o] *= er[r];   // diag(gamma) dO
                }
        }
        __syncthreads();
        {   // dS = Q^T diag(gamma) dO + gamma_C dS' - K^T diag(gamma) dR  (wave w: state rows SR0 ..)
            f32x4 a[NR][2], qt[2][NR], kt[2][NR], ob[2][2], rb[2][2];
#pragma unroll
            for (int x = 0; x < NR; ++x) a[x][0] = a[x][1] = z4;
            kpipe<KC>(
                [&](int u, int i) {
#pragma unroll
                    for (int x = 0; x < NR; ++x) {
                        qt[u][x] = kcol4(Qs, DP, SR0 + 16 * x + lr, 16 * i, lq);
                        kt[u][x] = kcol4(Ks, DP, SR0 + 16 * x + lr, 16 * i, lq);
                    }
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        ob[u][j] = kcol4(dOs, VP, 16 * j + lr, 16 * i, lq);
                        rb[u][j] = -kcol4(dRs, VP, 16 * j + lr, 16 * i, lq);
                    }
                },
                [&](int u, int) {
                    // diag(gamma) dO and dR are not bf16 values
                    const Op4<BF, false> o0 = op4<BF, false>(ob[u][0]), o1 = op4<BF, false>(ob[u][1]);
                    const Op4<BF, false> r0 = op4<BF, false>(rb[u][0]), r1 = op4<BF, false>(rb[u][1]);
#pragma unroll
                    for (int x = 0; x < NR; ++x) {
                        const auto qx = op4<BF, BF>(qt[u][x]), kx = op4<BF, BF>(kt[u][x]);
                        a[x][0] = mm4(mm4(a[x][0], qx, o0), kx, r0);
                        a[x][1] = mm4(mm4(a[x][1], qx, o1), kx, r1);
                    }
                });
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
    if (dstate_in) state_from_lds<D, BV, VP>(dstate_in + unit * D * D, dS, vb * BV);
}

// ---------------------------------------------------------------------------
// Per-chunk gradients.  The value dimension is walked in blocks of 16 columns;
// dQ, dK (C x D) and dP, dTm (C x C) accumulate in registers across blocks.
// Every product runs on the matrix cores in the inputs' precision (mm4: fp32
// instructions, or bf16 ones with split operands), one 16 x 16 output tile per
// instruction chain.
// Wave w owns rows 16w .. 16w + 15 (tokens) of every row-partitioned product;
// in a tile, lane l holds rows 4 (l / 16) + r, r < 4, of column l % 16.  The
// contraction runs in 16-wide k blocks: in product m of a block, lane l reads
// A(row l % 16, k = 4 (l / 16) + m) and B(k = 4 (l / 16) + m, column l % 16),
// so an operand row contiguous in k is one 16-byte read per block, and a
// column read touches rows 4 apart.  Row pitches: D + 4 for K and Q, 20 for
// value blocks, C + 4 for C x C matrices (four rows apart is 16 banks apart:
// column reads are conflict-free; 16-byte row reads are too).  The loads of a
// block are issued before the products of the previous one
// (sched_barrier keeps the compiler from sinking them to their use).
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
    constexpr int BV = 16, DP = D + 4, VP = BV + 4, CQ = BC + 4;
    constexpr int NJ = D / 16, NP = BC / 16;   // 16-column tiles of dQ/dK and of dP/dTm
    constexpr int KD = D / 16, KC = BC / 16;   // 16-wide k blocks over D and over C
    // bf16 inputs: bf16 matrix cores (K, Q exact; dO exact when it is bf16; the rest split)
    constexpr bool BF = sizeof(TI) == 2, OX = BF && sizeof(TO) == 2;
    static_assert(BNT == 256 && BC == 64, "four waves of 16 token rows");
    // phase-1 buffers (per value block) and phase-2 buffers (C x C) share one region
    constexpr int P1 = 2 * D * VP + 6 * BC * VP;
    constexpr int P2 = 3 * BC * CQ;
    constexpr int UN = P1 > P2 ? P1 : P2;
    // Pt holds P transposed (P is only read as P^T), then X = dP o P
    __shared__ __attribute__((aligned(16))) float Qs[BC * DP], Ks[BC * DP], un[UN], Ns[BC * CQ], Pt[BC * CQ], bt[BC];
    __shared__ float gq[BC], gk[BC], gd[BC], red[BNT], redb[BNT];
    __shared__ double g[BC];
    float *Sb = un, *dSb = Sb + D * VP, *Vb = dSb + D * VP, *dOb = Vb + BC * VP, *Rb = dOb + BC * VP,
          *Ub = Rb + BC * VP, *dUb = Ub + BC * VP, *dRb = dUb + BC * VP;
    float *X1 = un, *X2 = un + BC * CQ, *X3 = un + 2 * BC * CQ;

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
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    // row and column reads of a 16-wide k block (krow4, kcol4)
    auto row4 = [&](const float *m, int pitch, int r, int k0) { return krow4(m, pitch, r, k0, lq); };
    auto col4 = [&](const float *m, int pitch, int col, int k0) { return kcol4(m, pitch, col, k0, lq); };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    {
        Rows<D, TI> rk, rq;
        CCm nm, pm;
        rk.fetch(k + row0 * D, tok, n);
        rq.fetch(q + row0 * D, tok, n);
        nm.fetch(gc + G_FLOATS);
        pm.fetch(gc + G_FLOATS + BC * BC);
        rk.put(Ks, DP);
        rq.put(Qs, DP);
        // bf16 inputs: N and P^T as packed hi/lo words (split once for all waves and blocks)
        if constexpr (BF) {
            nm.put_packed(Ns, CQ);
            pm.put_t_packed(Pt, CQ);
        } else {
            nm.put(Ns, CQ);
            pm.put_t(Pt, CQ);
        }
    }
    if (tid < BC) {
        g[tid] = reinterpret_cast<const double *>(gc)[tid];
        bt[tid] = tid < n ? beta[row0 + (size_t)tid * H] : 0.f;
    }
    float sdot = 0.f;
    f32x4 aq[NJ], ak[NJ], ap[NP], at[NP];
#pragma unroll
    for (int j = 0; j < NJ; ++j) aq[j] = ak[j] = z4;
#pragma unroll
    for (int j = 0; j < NP; ++j) ap[j] = at[j] = z4;
    __syncthreads();
    const double gC = g[n - 1];
    const float ea = dexp2(g[ra], 0.0), eca = dexp2(gC, g[ra]);   // gamma, gamma_C / gamma of row ra
    // the same and beta for this lane's accumulator rows R0 + 4 (lane / 16) + r
    float er[4], ecr[4], br[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = R0 + 4 * lq + r;
        er[r] = dexp2(g[t], 0.0);
        ecr[r] = dexp2(gC, g[t]);
        br[r] = bt[t];
    }
    // gate row terms <dR, KS>, <U, KdS> of this lane's accumulator rows
    // t = R0 + 4 (lane / 16) + r: each lane sums its own column's products over
    // the value blocks; the 16 lanes of a row are reduced once at the end
    float gkr[4] = {0.f, 0.f, 0.f, 0.f}, gdr[4] = {0.f, 0.f, 0.f, 0.f};

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
            // bf16 inputs: S and dS' as packed hi/lo words
            *reinterpret_cast<f32x4 *>(&Sb[r * VP + cc]) = BF ? pack_hilo4(a) : a;
            *reinterpret_cast<f32x4 *>(&dSb[r * VP + cc]) = BF ? pack_hilo4(d2) : d2;
#pragma unroll
            for (int j = 0; j < 4; ++j) sdot = fmaf(a[j], d2[j], sdot);
        }
        rv.put(Vb, VP);
        ro.put(dOb, VP);
        if (vb + 1 < D / BV) fetch(vb + 1);
        __syncthreads();
        // KS = K S, KdS = K dS' (C x BV), kept in registers;  R = V - diag(gamma) KS
        // (two partial sums each, even and odd k blocks)
        f32x4 ks, kds;
        {
            f32x4 ks2[2] = {z4, z4}, kds2[2] = {z4, z4};
            f32x4 ka[2], sb[2], sd[2];
            auto ld = [&](int u, int kb) {
                ka[u] = row4(Ks, DP, ra, kb);
                sb[u] = col4(Sb, VP, lr, kb);
                sd[u] = col4(dSb, VP, lr, kb);
            };
            ld(0, 0);
#pragma unroll
            for (int i = 0; i < KD; ++i) {
                const int u = i & 1;
                if (i + 1 < KD) ld(u ^ 1, 16 * (i + 1));
                fence();
                const auto a = op4<BF, BF>(ka[u]);
                ks2[i & 1] = mm4(ks2[i & 1], a, op4_stored<BF>(sb[u]));
                kds2[i & 1] = mm4(kds2[i & 1], a, op4_stored<BF>(sd[u]));
                fence();
            }
            ks = ks2[0] + ks2[1];
            kds = kds2[0] + kds2[1];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = R0 + 4 * lq + r, o = t * VP + lr;
            Rb[o] = Vb[o] - er[r] * ks[r];
        }
        __syncthreads();
        // U = N diag(beta) R ; dU = P^T dO + diag(gamma_C/gamma) K dS'
        f32x4 u4;   // U, this lane's accumulator rows
        {
            f32x4 p1[2] = {z4, z4}, p2[2] = {z4, z4};   // two partial sums per product (k block even, odd)
            f32x4 na[2], pa[2], ba[2], rb[2], ob[2];
            auto ld = [&](int u, int kb) {
                na[u] = row4(Ns, CQ, ra, kb);
                pa[u] = row4(Pt, CQ, ra, kb);
                ba[u] = *reinterpret_cast<const f32x4 *>(&bt[kb + 4 * lq]);
                rb[u] = col4(Rb, VP, lr, kb);
                ob[u] = col4(dOb, VP, lr, kb);
            };
            ld(0, 0);
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                const int u = i & 1;
                if (i + 1 < KC) ld(u ^ 1, 16 * (i + 1));
                fence();
                p1[i & 1] = mm4(p1[i & 1], op4_stored<BF>(na[u]), op4<BF, false>(ba[u] * rb[u]));
                p2[i & 1] = mm4(p2[i & 1], op4_stored<BF>(pa[u]), op4<BF, OX>(ob[u]));
                fence();
            }
            u4 = p1[0] + p1[1];
            const f32x4 a2 = p2[0] + p2[1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = R0 + 4 * lq + r, o = t * VP + lr;
                Ub[o] = u4[r];
                dUb[o] = fmaf(ecr[r], kds[r], a2[r]);
            }
        }
        __syncthreads();
        {   // dR = diag(beta) N^T dU  (= dV)
            f32x4 p1[2] = {z4, z4};
            f32x4 na[2], db[2];
            auto ld = [&](int u, int kb) {
                na[u] = col4(Ns, CQ, ra, kb);
                db[u] = col4(dUb, VP, lr, kb);
            };
            ld(0, 0);
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                const int u = i & 1;
                if (i + 1 < KC) ld(u ^ 1, 16 * (i + 1));
                fence();
                p1[i & 1] = mm4(p1[i & 1], op4_stored<BF>(na[u]), op4<BF, false>(db[u]));
                fence();
            }
            const f32x4 a1 = p1[0] + p1[1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = R0 + 4 * lq + r;
                const float x = br[r] * a1[r];
                dRb[t * VP + lr] = x;
                if (t < n) dv[(row0 + (size_t)t * H) * D + vb * BV + lr] = x;
                gkr[r] = fmaf(x, ks[r], gkr[r]);
                gdr[r] = fmaf(u4[r], kds[r], gdr[r]);
            }
        }
        __syncthreads();
        // register accumulations over this value block (k = value column s)
        //   dQ += dO S^T (rows scaled by gamma after the last block) ;
        //   dK += diag(gamma_C/gamma) U dS'^T - diag(gamma) dR S^T ; dP += dO U^T ; dTm += dU R^T
        {
            const auto o4 = op4<BF, OX>(row4(dOb, VP, ra, 0));
            const auto du4 = op4<BF, false>(row4(dUb, VP, ra, 0));
            const auto ua4 = op4<BF, false>(eca * row4(Ub, VP, ra, 0));
            const auto ra4 = op4<BF, false>(-ea * row4(dRb, VP, ra, 0));
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const auto sq = op4_stored<BF>(row4(Sb, VP, 16 * j + lr, 0));
                const auto sd = op4_stored<BF>(row4(dSb, VP, 16 * j + lr, 0));
                aq[j] = mm4(aq[j], o4, sq);
                ak[j] = mm4(mm4(ak[j], ua4, sd), ra4, sq);
            }
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                ap[j] = mm4(ap[j], o4, op4<BF, false>(row4(Ub, VP, 16 * j + lr, 0)));
                at[j] = mm4(at[j], du4, op4<BF, false>(row4(Rb, VP, 16 * j + lr, 0)));
            }
        }
        __syncthreads();
    }

    // gamma <dO, Q S> of row t is <Q_t, (diag(gamma) dO S^T)_t>, and the second
    // factor is what dQ holds after the value blocks and the row scaling
    float gqv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = R0 + 4 * lq + r;
#pragma unroll
        for (int j = 0; j < NJ; ++j) aq[j][r] *= er[r];
        float x = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) x = fmaf(Qs[t * DP + 16 * j + lr], aq[j][r], x);
        gqv[r] = row16_sum(x);
    }

    // ---- phase 2: C x C algebra (buffers X1..X3 replace the value-block buffers) ----
    // (a) X1 = dP o Gam (lower incl, rows < n), X2 = dTm, X3 = Q K^T
    {
        f32x4 qk[NP];
#pragma unroll
        for (int j = 0; j < NP; ++j) qk[j] = z4;
        f32x4 qa[2], kb4[2][NP];
        auto ld = [&](int u, int kb) {
            qa[u] = row4(Qs, DP, ra, kb);
#pragma unroll
            for (int j = 0; j < NP; ++j) kb4[u][j] = row4(Ks, DP, 16 * j + lr, kb);
        };
        ld(0, 0);
#pragma unroll
        for (int i = 0; i < KD; ++i) {
            const int u = i & 1;
            if (i + 1 < KD) ld(u ^ 1, 16 * (i + 1));
            fence();
            const auto a = op4<BF, BF>(qa[u]);
#pragma unroll
            for (int j = 0; j < NP; ++j) qk[j] = mm4(qk[j], a, op4<BF, BF>(kb4[u][j]));
            fence();
        }
#pragma unroll
        for (int j = 0; j < NP; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = R0 + 4 * lq + r, s = 16 * j + lr;
                const float gam = materialize(dexp2(g[t], g[min(s, t)]));
                X1[t * CQ + s] = (s <= t && t < n) ? ap[j][r] * gam : 0.f;
                X2[t * CQ + s] = at[j][r];
                X3[t * CQ + s] = qk[j][r];
            }
    }
    __syncthreads();
    // (b) dQ += (dP o Gam) K ; dK += (dP o Gam)^T Q ; X = dP o P = X1 o QK^T into Pt
    //     (P is no longer needed) ; dbeta from Tm = N diag(beta): sum_s dTm_st N_st
    {
        // steps (k block, tile j); the operands of step i + 1 load during step i
        f32x4 xa[2], xt[2], kv[2], qv[2];
        Op4<BF, false> xo, xto;   // the current k block's X1 operands, converted once
        auto ld = [&](int u, int i) {
            const int kb = 16 * (i / NJ), j = i % NJ;
            if (j == 0) {
                xa[(i / NJ) & 1] = row4(X1, CQ, ra, kb);
                xt[(i / NJ) & 1] = col4(X1, CQ, ra, kb);
            }
            kv[u] = col4(Ks, DP, 16 * j + lr, kb);
            qv[u] = col4(Qs, DP, 16 * j + lr, kb);
        };
        ld(0, 0);
#pragma unroll
        for (int i = 0; i < KC * NJ; ++i) {
            const int u = i & 1, w = (i / NJ) & 1, j = i % NJ;
            if (i + 1 < KC * NJ) ld(u ^ 1, i + 1);
            fence();
            if (j == 0) {
                xo = op4<BF, false>(xa[w]);
                xto = op4<BF, false>(xt[w]);
            }
            aq[j] = mm4(aq[j], xo, op4<BF, BF>(kv[u]));
            ak[j] = mm4(ak[j], xto, op4<BF, BF>(qv[u]));
            fence();
        }
    }
    for (int idx = tid; idx < BC * BC; idx += BNT) {
        const int t = idx / BC, s = idx % BC;
        Pt[t * CQ + s] = X1[t * CQ + s] * X3[t * CQ + s];
    }
    // dbeta of token t = lane: wave w sums s = w (mod 4); the four are added at the end
    const int wv = tid >> 6;
    float dbt = 0.f;
#pragma unroll 4
    for (int s = wv; s < BC; s += 4) {
        const float nv = BF ? unpack_hilo(Ns[s * CQ + lane]) : Ns[s * CQ + lane];
        dbt = fmaf(X2[s * CQ + lane], nv, dbt);
    }
    __syncthreads();
    // (c) T1 = N^T dTm diag(beta) into X1 ; X3 = K K^T
    {
        f32x4 a[NP], kk4[NP];
#pragma unroll
        for (int j = 0; j < NP; ++j) a[j] = kk4[j] = z4;
        f32x4 na[2], xb[2][NP];
        auto ld = [&](int u, int kb) {
            na[u] = col4(Ns, CQ, ra, kb);
#pragma unroll
            for (int j = 0; j < NP; ++j) xb[u][j] = col4(X2, CQ, 16 * j + lr, kb);
        };
        ld(0, 0);
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int u = i & 1;
            if (i + 1 < KC) ld(u ^ 1, 16 * (i + 1));
            fence();
            const auto a0 = op4_stored<BF>(na[u]);
#pragma unroll
            for (int j = 0; j < NP; ++j) a[j] = mm4(a[j], a0, op4<BF, false>(xb[u][j]));
            fence();
        }
        f32x4 ka[2], kb4[2][NP];
        auto ldk = [&](int u, int kb) {
            ka[u] = row4(Ks, DP, ra, kb);
#pragma unroll
            for (int j = 0; j < NP; ++j) kb4[u][j] = row4(Ks, DP, 16 * j + lr, kb);
        };
        ldk(0, 0);
#pragma unroll
        for (int i = 0; i < KD; ++i) {
            const int u = i & 1;
            if (i + 1 < KD) ldk(u ^ 1, 16 * (i + 1));
            fence();
            const auto a0 = op4<BF, BF>(ka[u]);
#pragma unroll
            for (int j = 0; j < NP; ++j) kk4[j] = mm4(kk4[j], a0, op4<BF, BF>(kb4[u][j]));
            fence();
        }
#pragma unroll
        for (int j = 0; j < NP; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = R0 + 4 * lq + r, s = 16 * j + lr;
                X1[t * CQ + s] = a[j][r] * bt[s];
                X3[t * CQ + s] = kk4[j][r];
            }
    }
    __syncthreads();
    // (d) dA = -T1 N^T, strict lower part, into X2
    {
        f32x4 a[NP];
#pragma unroll
        for (int j = 0; j < NP; ++j) a[j] = z4;
        f32x4 xa[2], nb[2][NP];
        auto ld = [&](int u, int kb) {
            xa[u] = row4(X1, CQ, ra, kb);
#pragma unroll
            for (int j = 0; j < NP; ++j) nb[u][j] = row4(Ns, CQ, 16 * j + lr, kb);
        };
        ld(0, 0);
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int u = i & 1;
            if (i + 1 < KC) ld(u ^ 1, 16 * (i + 1));
            fence();
            const auto a0 = op4<BF, false>(xa[u]);
#pragma unroll
            for (int j = 0; j < NP; ++j) a[j] = mm4(a[j], a0, op4_stored<BF>(nb[u][j]));
            fence();
        }
#pragma unroll
        for (int j = 0; j < NP; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = R0 + 4 * lq + r, s = 16 * j + lr;
                X2[t * CQ + s] = s < t ? -a[j][r] : 0.f;
            }
    }
    __syncthreads();
    // (e) E = dA beta_t Gam (strict lower); X1 = E + E^T ; X += dA o A
    //     (A = beta_t K K^T Gam) ; dbeta from A: sum_s dA_ts (k_t . k_s) Gam_ts
    for (int idx = tid; idx < BC * BC; idx += BNT) {
        const int t = idx / BC, s = idx % BC;
        const float gfull = materialize(dexp2(g[t], g[s]));   // every element, then selected
        const float gts = s < t ? gfull : 0.f;
        const float kg = X3[t * CQ + s] * gts;
        const float e = X2[t * CQ + s] * bt[t] * gts;
        if (s < t) X1[s * CQ + t] = e;
        if (s <= t) X1[t * CQ + s] = e;
        Pt[t * CQ + s] = fmaf(X2[t * CQ + s], bt[t] * kg, Pt[t * CQ + s]);
    }
    // the same terms in the same order as a loop over s < lane, taken for every
    // s and selected, so no lane waits behind another's loads
    for (int s = wv; s < BC; s += 4) {
        const float v = materialize(fmaf(X2[lane * CQ + s], X3[lane * CQ + s] * dexp2(g[lane], g[s]), dbt));
        dbt = s < lane ? v : dbt;
    }
    __syncthreads();
    // (f) dK += (E + E^T) K
    {
        f32x4 xa[2], kv[2];
        Op4<BF, false> xo;
        auto ld = [&](int u, int i) {
            const int kb = 16 * (i / NJ), j = i % NJ;
            if (j == 0) xa[(i / NJ) & 1] = row4(X1, CQ, ra, kb);
            kv[u] = col4(Ks, DP, 16 * j + lr, kb);
        };
        ld(0, 0);
#pragma unroll
        for (int i = 0; i < KC * NJ; ++i) {
            const int u = i & 1, w = (i / NJ) & 1, j = i % NJ;
            if (i + 1 < KC * NJ) ld(u ^ 1, i + 1);
            fence();
            if (j == 0) xo = op4<BF, false>(xa[w]);
            ak[j] = mm4(ak[j], xo, op4<BF, BF>(kv[u]));
            fence();
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
#pragma unroll
    for (int r = 0; r < 4; ++r) {   // gamma <dO, QS>, -gamma <dR, KS>, (gamma_C/gamma) <U, KdS>
        const int t = R0 + 4 * lq + r;
        const float x2 = row16_sum(gkr[r]), x3 = row16_sum(gdr[r]);
        if (lr == 0) {
            gq[t] = gqv[r];
            gk[t] = -er[r] * x2;
            gd[t] = ecr[r] * x3;
        }
    }
    // gate (wave 0, thread j = token j of the chunk).  The pairs i < j <= t of X
    // (lower triangular, rows >= n zero): column suffix sums over t in place
    // (lane i walks column i), then lane j adds row j over i < j.
    if (tid < BC) {
        float acc = 0.f;
#pragma unroll 8
        for (int t = BC - 1; t >= 0; --t) {
            acc += Pt[t * CQ + tid];
            Pt[t * CQ + tid] = acc;
        }
    }
    red[tid] = sdot;
    redb[tid] = dbt;
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
        for (int i = 0; i < BC; ++i) {
            const float v = Pt[j * CQ + i];
            cross += i < j ? v : 0.f;
        }
        if (j < n) {
            dlog_alpha[row0 + (size_t)j * H] = suf + pre + cross + dexp2(gC, 0.0) * x;
            dbeta[row0 + (size_t)j * H] = (redb[j] + redb[j + 64]) + (redb[j + 128] + redb[j + 192]);
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
