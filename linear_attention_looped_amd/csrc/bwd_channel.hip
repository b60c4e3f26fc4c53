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
// One workgroup of 8 waves per (b, h, 16-column block); each wave owns 2 state
// columns and every row (lane l: rows RPL l .. RPL l + RPL - 1, RPL = d/64), so
// sums over rows are wave reductions.  The workgroup first runs the recurrence
// forward and stores the state entering every segment of 16 tokens; then, for
// the segments in reverse order, it recomputes the segment's 17 states into
// registers and walks its tokens backwards.  Per token the row quantities of
// the workgroup's 16 columns are summed in LDS (float atomics from the 8
// waves) and written once per segment to a partial buffer per column block,
// which a second kernel sums.  Inputs of a segment are staged in LDS as fp32.
#include "common.h"
#include "internal.h"

namespace lt2 {

namespace {

constexpr int KS = 16;               // segment (checkpoint interval) in tokens
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

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <typename T>
__device__ __forceinline__ float ld1(const T *p);
template <>
__device__ __forceinline__ float ld1<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float ld1<uint16_t>(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }

template <int D, typename TI, typename TO>
__global__ __launch_bounds__(KNT) void kda_bwd_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                       const TI *__restrict__ v, const float *__restrict__ alpha,
                                                       const float *__restrict__ beta, const float *state_in,
                                                       const TO *__restrict__ dout, const float *dstate_out,
                                                       float *__restrict__ dv_out, float *dstate_in,
                                                       float *__restrict__ ck, float *__restrict__ part, int B, int L,
                                                       int H) {
    constexpr int RPL = D / 64;      // rows per lane
    constexpr int NCB = D / KBV;
    __shared__ float sk[KS][D], sq[KS][D], sa[KS][D];
    __shared__ float sv[KS][KBV], sd[KS][KBV], sb[KS];
    __shared__ float acc[KS][3][D];  // per token of the segment: dq, dk, d(log alpha) row sums
    __shared__ float accb[KS];

    const int cb = blockIdx.x % NCB;
    const size_t unit = blockIdx.x / NCB;
    const int h = (int)(unit % H), b = (int)(unit / H);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cw = KCOL * wave;              // this wave's first column inside the block
    const int c0 = cb * KBV + cw;            // ... in the state
    const int r0 = RPL * lane;               // this lane's first row
    const int NS = (L + KS - 1) / KS;
    const size_t n_tok = (size_t)B * L * H;
    float *ckp = ck + unit * (size_t)NS * D * D;

    auto tok_of = [&](int t) __attribute__((always_inline)) { return ((size_t)b * L + t) * H + h; };
    // Inputs of tokens t0 .. t0 + KS - 1 (rows past L: k = q = 0, alpha = 1, beta = 0, v = dO = 0).
    auto stage = [&](int t0) __attribute__((always_inline)) {
        for (int idx = tid; idx < KS * D; idx += KNT) {
            const int tt = idx / D, c = idx % D, t = t0 + tt;
            const bool ok = t < L;
            const size_t o = tok_of(ok ? t : 0) * D + c;
            sk[tt][c] = ok ? ld1<TI>(k + o) : 0.f;
            sq[tt][c] = ok ? ld1<TI>(q + o) : 0.f;
            sa[tt][c] = ok ? alpha[o] : 1.f;
        }
        for (int idx = tid; idx < KS * KBV; idx += KNT) {
            const int tt = idx / KBV, c = idx % KBV, t = t0 + tt;
            const bool ok = t < L;
            const size_t o = tok_of(ok ? t : 0) * D + cb * KBV + c;
            sv[tt][c] = ok ? ld1<TI>(v + o) : 0.f;
            sd[tt][c] = ok ? ld1<TO>(dout + o) : 0.f;
        }
        if (tid < KS) {
            const int t = t0 + tid;
            sb[tid] = t < L ? beta[tok_of(t)] : 0.f;
        }
    };
    // One forward token on the wave's state slice; returns y = S^T k (in y).
    auto step = [&](float (&S)[RPL][KCOL], float (&y)[KCOL], int tt) __attribute__((always_inline)) {
        float kr[RPL], ar[RPL];
#pragma unroll
        for (int i = 0; i < RPL; ++i) { kr[i] = sk[tt][r0 + i]; ar[i] = sa[tt][r0 + i]; }
        const float bt = sb[tt];
#pragma unroll
        for (int j = 0; j < KCOL; ++j) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) p += kr[i] * S[i][j];
            y[j] = wave_sum(p);
        }
#pragma unroll
        for (int j = 0; j < KCOL; ++j) {
            const float vj = sv[tt][cw + j];
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const float bk = bt * kr[i];
                S[i][j] = ar[i] * (S[i][j] - bk * y[j]) + bk * vj;
            }
        }
    };

    // ---- forward: the state entering every segment ----
    float S[RPL][KCOL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int j = 0; j < KCOL; ++j) S[i][j] = state_in ? state_in[(unit * D + r0 + i) * D + c0 + j] : 0.f;
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int j = 0; j < KCOL; ++j) ckp[((size_t)s * D + r0 + i) * D + c0 + j] = S[i][j];
        __syncthreads();   // the previous segment's inputs are no longer read
        stage(s * KS);
        __syncthreads();
        const int n = min(KS, L - s * KS);
        for (int tt = 0; tt < n; ++tt) {
            float y[KCOL];
            step(S, y, tt);
        }
    }

    // ---- backward, segments in reverse ----
    float G[RPL][KCOL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int j = 0; j < KCOL; ++j) G[i][j] = dstate_out ? dstate_out[(unit * D + r0 + i) * D + c0 + j] : 0.f;
    for (int s = NS - 1; s >= 0; --s) {
        const int t0 = s * KS;
        const int n = min(KS, L - t0);
        __syncthreads();   // the previous segment's inputs and sums have been read
        stage(t0);
        for (int idx = tid; idx < KS * 3 * D; idx += KNT) (&acc[0][0][0])[idx] = 0.f;
        if (tid < KS) accb[tid] = 0.f;
        __syncthreads();
        // states before each token of the segment and after its last: Sx[tt] = S_{t0+tt-1}
        float Sx[KS + 1][RPL][KCOL], yy[KS][KCOL];
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int j = 0; j < KCOL; ++j) Sx[0][i][j] = ckp[((size_t)s * D + r0 + i) * D + c0 + j];
#pragma unroll
        for (int tt = 0; tt < KS; ++tt) {
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int j = 0; j < KCOL; ++j) Sx[tt + 1][i][j] = Sx[tt][i][j];
            if (tt < n) step(Sx[tt + 1], yy[tt], tt);
        }
#pragma unroll
        for (int tt = KS - 1; tt >= 0; --tt) {
            if (tt >= n) continue;
            float kr[RPL], qr[RPL], ar[RPL], vj[KCOL], dj[KCOL];
#pragma unroll
            for (int i = 0; i < RPL; ++i) { kr[i] = sk[tt][r0 + i]; qr[i] = sq[tt][r0 + i]; ar[i] = sa[tt][r0 + i]; }
#pragma unroll
            for (int j = 0; j < KCOL; ++j) { vj[j] = sv[tt][cw + j]; dj[j] = sd[tt][cw + j]; }
            const float bt = sb[tt];
            float dE[RPL][KCOL], red[2 * KCOL + 1];
            float dq_[RPL], dla[RPL], gv[RPL];
#pragma unroll
            for (int j = 0; j < 2 * KCOL + 1; ++j) red[j] = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                dq_[i] = 0.f; dla[i] = 0.f; gv[i] = 0.f;
                const float bk = bt * kr[i];
#pragma unroll
                for (int j = 0; j < KCOL; ++j) {
                    G[i][j] += qr[i] * dj[j];
                    dq_[i] += Sx[tt + 1][i][j] * dj[j];
                    // E = S_{t-1} - beta k y^T: exact zero gradient for alpha = 0 and no
                    // cancellation for small alpha (unlike S_t - beta k v^T = alpha E)
                    dla[i] += G[i][j] * (Sx[tt][i][j] - bk * yy[tt][j]);
                    dE[i][j] = ar[i] * G[i][j];
                    gv[i] += G[i][j] * vj[j];
                    red[j] += dE[i][j] * kr[i];              // z_j
                    red[KCOL + j] += G[i][j] * kr[i];        // dv_j / beta
                    red[2 * KCOL] += kr[i] * (G[i][j] * vj[j] - dE[i][j] * yy[tt][j]);   // dbeta
                }
                dla[i] *= ar[i];
            }
#pragma unroll
            for (int j = 0; j < 2 * KCOL + 1; ++j) red[j] = wave_sum(red[j]);
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                float dk_ = gv[i];
#pragma unroll
                for (int j = 0; j < KCOL; ++j) {
                    dk_ -= Sx[tt][i][j] * red[j] + dE[i][j] * yy[tt][j];
                    G[i][j] = dE[i][j] - bt * kr[i] * red[j];
                }
                atomicAdd(&acc[tt][0][r0 + i], dq_[i]);
                atomicAdd(&acc[tt][1][r0 + i], bt * dk_);
                atomicAdd(&acc[tt][2][r0 + i], dla[i]);
            }
            if (lane == 0) atomicAdd(&accb[tt], red[2 * KCOL]);
            if (lane < KCOL) {
                const float dvv = bt * (lane == 0 ? red[KCOL] : red[KCOL + 1]);
                dv_out[tok_of(t0 + tt) * D + c0 + lane] = dvv;
            }
        }
        __syncthreads();
        // this block's partial row sums of the segment's tokens
        float *pb = part + (size_t)cb * (3 * n_tok * D + n_tok);
        for (int idx = tid; idx < n * 3 * D; idx += KNT) {
            const int tt = idx / (3 * D), rem = idx % (3 * D), qd = rem / D, c = rem % D;
            pb[(size_t)qd * n_tok * D + tok_of(t0 + tt) * D + c] = acc[tt][qd][c];
        }
        if (tid < n) pb[3 * n_tok * D + tok_of(t0 + tid)] = accb[tid];
    }
    if (dstate_in) {
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int j = 0; j < KCOL; ++j) dstate_in[(unit * D + r0 + i) * D + c0 + j] = G[i][j];
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
    const unsigned blocks = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
    hipLaunchKernelGGL(kda_bwd_reduce_kernel, dim3(blocks), dim3(256), 0, s, part, D / KBV, n_tok, D, a.dq, a.dk,
                       a.dlog_alpha, a.dbeta);
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
