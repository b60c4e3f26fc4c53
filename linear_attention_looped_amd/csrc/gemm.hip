// gemm.hip -- bf16 matrix-core GEMM with the looped block's fused epilogues.
//
//   C[m][n] = sum_k A[m][k] * B[n][k]        (A: [M, K], B: [N, K], both K-contiguous)
//
// which is y = x W^T for weights stored [d_out, d_in].  Workgroup tile 256 x 128
// x 64, four waves, each wave 64 rows x 128 columns (4 x 8 tiles of
// v_mfma_f32_16x16x32_bf16).  A and B tiles are double-buffered in LDS; the
// next K-tile's global loads are in flight while the current one computes.
//
// Epilogues (one launch each, fused into the store):
//   EPI_PROJ  input projection of the looped block: columns [0, H*d) -> q and
//             [H*d, 2H*d) -> k, each L2-normalised per head (x / max(|x|, 1e-6))
//             and stored bf16; [2H*d, 3H*d) -> v (bf16); [3H*d, 3H*d + H) ->
//             beta = sigmoid(z); [3H*d + H, 3H*d + 2H) -> alpha = exp(-softplus(z))
//             (both fp32, one per head).
//   EPI_RESID residual update h[m][n] += C[m][n] (fp32), and xb[m][n] = bf16(h),
//             the next loop's GEMM input.
#include "common.h"
#include "gemm.h"

namespace lt2 {

namespace {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int PITCH = BK + 8;   // bf16 elements per LDS row (16-byte aligned, staggered banks)

struct ProjOut {
    uint16_t *q, *k, *v;   // [M, H*d] bf16
    float *beta, *alpha;   // [M, H]
    int H, d;
};

struct ResidOut {
    float *h;              // [M, N] fp32, updated in place
    uint16_t *xb;          // [M, N] bf16 copy
};

__device__ __forceinline__ float sigmoidf_acc(float z) { return 1.f / (1.f + expf(-z)); }

template <int EPI, int DH>
__global__ __launch_bounds__(256) void gemm_bf16_nt_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                                                           int M, int N, int K, int lda, int ldb, ProjOut po,
                                                           ResidOut ro) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * PITCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const int n_tiles = (N + BN - 1) / BN;
    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    const int mt = logical / n_tiles, nt = logical % n_tiles;
    const int m0 = mt * BM, n0 = nt * BN;

    // global -> register staging: A 8 x 16 bytes, B 4 x 16 bytes per lane
    // (plain macros rather than lambdas: a captured array would be moved to LDS)
    uint4 ra[8], rb[4];
#define LT2_GEMM_LOAD(k0)                                                                        \
    do {                                                                                         \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                          \
            const int c = tid + 256 * i;                                                         \
            const int gm = min(m0 + (c >> 3), M - 1);                                            \
            ra[i] = *reinterpret_cast<const uint4 *>(A + (size_t)gm * lda + (k0) + 8 * (c & 7)); \
        }                                                                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                          \
            const int c = tid + 256 * i;                                                         \
            const int gn = min(n0 + (c >> 3), N - 1);                                            \
            rb[i] = *reinterpret_cast<const uint4 *>(B + (size_t)gn * ldb + (k0) + 8 * (c & 7)); \
        }                                                                                        \
    } while (0)
#define LT2_GEMM_STORE(buf)                                                                      \
    do {                                                                                         \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                          \
            const int c = tid + 256 * i;                                                         \
            *reinterpret_cast<uint4 *>(&As[buf][(c >> 3) * PITCH + 8 * (c & 7)]) = ra[i];         \
        }                                                                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                          \
            const int c = tid + 256 * i;                                                         \
            *reinterpret_cast<uint4 *>(&Bs[buf][(c >> 3) * PITCH + 8 * (c & 7)]) = rb[i];         \
        }                                                                                        \
    } while (0)

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = K / BK;
    LT2_GEMM_LOAD(0);
    LT2_GEMM_STORE(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) LT2_GEMM_LOAD((kt + 1) * BK);
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            bf16x8 a[4], b[8];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const bf16x8 *>(&As[buf][(64 * wave + 16 * i + lr) * PITCH + 32 * s + 8 * lq]);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[buf][(16 * j + lr) * PITCH + 32 * s + 8 * lq]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) {
            wait_vmem_all();
            LT2_GEMM_STORE(buf ^ 1);
        }
        __syncthreads();
    }

#undef LT2_GEMM_LOAD
#undef LT2_GEMM_STORE

    // ---- epilogue: lane holds C[m0 + 64 wave + 16 i + 4 lq + r][n0 + 16 j + lr] ----
    if constexpr (EPI == EPI_PROJ) {
        const int Hd = po.H * po.d;
        if (n0 < 3 * Hd) {
            // q, k or v block; a 128-column tile holds whole heads (Hd % 128 == 0)
            const int region = n0 / Hd;             // 0 q, 1 k, 2 v
            uint16_t *dst = region == 0 ? po.q : (region == 1 ? po.k : po.v);
            const int c0 = n0 - region * Hd;
            constexpr int TPH = DH / 16;            // column tiles per head
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + 64 * wave + 16 * i + 4 * lq + r;
                    float scale[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) scale[j] = 1.f;
                    if (region < 2) {
                        // per-head sum of squares: own tiles, then across the 16 lanes of the row
#pragma unroll
                        for (int h0 = 0; h0 < 8; h0 += TPH) {
                            float ss = 0.f;
#pragma unroll
                            for (int j = h0; j < h0 + TPH; ++j) ss += acc[i][j][r] * acc[i][j][r];
                            ss += __shfl_xor(ss, 1);
                            ss += __shfl_xor(ss, 2);
                            ss += __shfl_xor(ss, 4);
                            ss += __shfl_xor(ss, 8);
                            const float sc = 1.f / fmaxf(sqrtf(ss), 1e-6f);
#pragma unroll
                            for (int j = h0; j < h0 + TPH; ++j) scale[j] = sc;
                        }
                    }
                    if (m < M) {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            dst[(size_t)m * Hd + c0 + 16 * j + lr] = bf16_bits(acc[i][j][r] * scale[j]);
                    }
                }
            }
        } else {
            // gate columns: beta (first H) and alpha (next H)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = m0 + 64 * wave + 16 * i + 4 * lq + r;
                        const int c = n0 + 16 * j + lr - 3 * Hd;
                        if (m >= M || c >= 2 * po.H) continue;
                        const float z = acc[i][j][r];
                        if (c < po.H) po.beta[(size_t)m * po.H + c] = sigmoidf_acc(z);
                        else po.alpha[(size_t)m * po.H + c - po.H] = sigmoidf_acc(-z);  // exp(-softplus(z))
                    }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + 64 * wave + 16 * i + 4 * lq + r;
                    const int n = n0 + 16 * j + lr;
                    if (m >= M || n >= N) continue;
                    const size_t o = (size_t)m * N + n;
                    const float hn = ro.h[o] + acc[i][j][r];
                    ro.h[o] = hn;
                    ro.xb[o] = bf16_bits(hn);
                }
    }
}

}  // namespace

hipError_t launch_gemm_proj(const uint16_t *X, const uint16_t *W, int M, int N, int K, uint16_t *q, uint16_t *k,
                            uint16_t *v, float *beta, float *alpha, int H, int d, hipStream_t s) {
    ProjOut po{q, k, v, beta, alpha, H, d};
    ResidOut ro{nullptr, nullptr};
    const unsigned grid = (unsigned)((M + BM - 1) / BM) * (unsigned)((N + BN - 1) / BN);
    if (d == 64)
        hipLaunchKernelGGL((gemm_bf16_nt_kernel<EPI_PROJ, 64>), dim3(grid), dim3(256), 0, s, X, W, M, N, K, K, K, po, ro);
    else
        hipLaunchKernelGGL((gemm_bf16_nt_kernel<EPI_PROJ, 128>), dim3(grid), dim3(256), 0, s, X, W, M, N, K, K, K, po, ro);
    return hipGetLastError();
}

hipError_t launch_gemm_resid(const uint16_t *O, const uint16_t *W, int M, int N, int K, float *h, uint16_t *xb,
                             hipStream_t s) {
    ProjOut po{};
    ResidOut ro{h, xb};
    const unsigned grid = (unsigned)((M + BM - 1) / BM) * (unsigned)((N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_bf16_nt_kernel<EPI_RESID, 128>), dim3(grid), dim3(256), 0, s, O, W, M, N, K, K, K, po, ro);
    return hipGetLastError();
}

// h_out = h_in (when distinct), xb = bf16(h_in)
__global__ __launch_bounds__(256) void cast_residual_kernel(const float *__restrict__ h_in, float *__restrict__ h_out,
                                                            uint16_t *__restrict__ xb, size_t n4) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 x = reinterpret_cast<const float4 *>(h_in)[i];
        if (h_out != h_in) reinterpret_cast<float4 *>(h_out)[i] = x;
        uint2 u;
        u.x = (uint32_t)bf16_bits(x.x) | ((uint32_t)bf16_bits(x.y) << 16);
        u.y = (uint32_t)bf16_bits(x.z) | ((uint32_t)bf16_bits(x.w) << 16);
        reinterpret_cast<uint2 *>(xb)[i] = u;
    }
}

hipError_t launch_cast_residual(const float *h_in, float *h_out, uint16_t *xb, size_t n, hipStream_t s) {
    const size_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192);
    hipLaunchKernelGGL(cast_residual_kernel, dim3(blocks), dim3(256), 0, s, h_in, h_out, xb, n4);
    return hipGetLastError();
}

}  // namespace lt2
