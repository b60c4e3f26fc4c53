// gemm.hip -- bf16 matrix-core GEMM with the looped block's fused epilogues.
//
//   C[m][n] = sum_k A[m][k] * B[n][k]        (A: [M, K], B: [N, K], both K-contiguous)
//
// which is y = x W^T for weights stored [d_out, d_in].  Workgroup tile 256 x 256
// x 64, eight waves, each wave 64 x 128 as 2 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 (128 accumulators per lane, so two waves share a
// SIMD and one wave's products run while the other waits on its LDS reads).
// Per k-step of 16 a wave reads two A and four B fragments for eight products.
// (A four-wave form with 128 x 128 wave tiles, one wave per SIMD, reads a third
// less LDS per product but leaves the matrix pipe idle on every LDS round trip;
// it stays available as the NW = 4 instance.)  A and B K-tiles are loaded
// straight into double-buffered LDS by LDS-DMA buffer loads; the workgroup
// meets once per K-tile, before its last k-step, so that k-step's products
// cover the next tile's first fragment reads.  LDS rows are 128 bytes with the
// 16-byte segments XOR-swizzled by row, so fragment reads of 8 or 16
// consecutive rows hit distinct banks.  The epilogues stage row blocks of the
// accumulators through the idle K-tile buffers and work row by row.
//
// For the few rows of a decode step (M of a few hundred) a 64 x 128 variant
// streams its K-tiles through five LDS stages instead (gemm_small_kernel).
//
// 32x32x16 operand layout: A[i][k]: lane = i + 32*(k/8), slot k%8; B[k][j]:
// lane = j + 32*(k/8), slot k%8; accumulator register r of lane l holds
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
//
// Epilogues (fused into the store):
//   EPI_PROJ  input projection of a looped layer: columns [0, H*d) -> q and
//             [H*d, 2H*d) -> k, for a gated-delta layer each L2-normalised per
//             head (x / max(|x|, 1e-6)), stored bf16; [2H*d, 3H*d) -> v (bf16);
//             with the output gate [3H*d, 4H*d) -> g = sigmoid(z) (bf16); for a
//             gated-delta layer the next H columns -> beta = sigmoid(z), the H
//             after them -> alpha = exp(-softplus(z)) (both fp32, one per head).
//   EPI_RESID residual update h[m][n] += C[m][n] (fp32), and xb[m][n] = bf16(h),
//             the next loop's GEMM input.
#include <type_traits>

#include "common.h"
#include "gemm.h"
#include "internal.h"

namespace lt2 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int GEMM_NW = 8;   // waves of the large-tile kernel
constexpr int SHORT_M = 64;  // rows of a short tile

// Tiles of the large kernel: full 256 x 256 tiles of the columns below N's last
// multiple of 256, then, when the columns left over are 32 or fewer (the
// projection's gate-transform columns), 64-row short tiles of those columns:
// such a column tile costs a whole tile's K loop of A (its products are few),
// and 64-row pieces spread that stream over four times as many compute units.
// Otherwise the last column tile is an ordinary (partial) one.  The short
// tiles take the block indices after the full tiles', which the hardware
// deals round-robin to the XCDs, so every XCD gets its share of both kinds.
__host__ __device__ inline bool gemm_short_cols(int N) { return N % BN != 0 && N % BN <= 32; }
__host__ __device__ inline int gemm_full_col_tiles(int N) {
    return gemm_short_cols(N) ? N / BN : (N + BN - 1) / BN;
}
inline unsigned gemm_grid(int M, int N) {
    const unsigned g = (unsigned)((M + BM - 1) / BM) * (unsigned)gemm_full_col_tiles(N);
    return gemm_short_cols(N) ? g + (unsigned)((M + SHORT_M - 1) / SHORT_M) : g;
}

typedef __attribute__((ext_vector_type(16))) float f32x16;

struct ProjOut {
    uint16_t *q, *k, *v;   // [M, H*d] bf16
    uint16_t *g;           // [M, H*d] bf16 output gate, or nullptr
    float *beta, *alpha;   // [M, H], or nullptr (no gate-transform columns)
    int H, d;
    int norm;              // L2-normalise q and k per head
};

struct ResidOut {
    float *h;              // [M, N] fp32, updated in place
    uint16_t *xb;          // [M, N] bf16 copy
};

// sigmoid(z) = 1 / (1 + 2^(-z log2 e)) on the hardware exp2 and reciprocal
// (each within about 1 ulp, no range branches; z -> -inf gives 1 / inf = 0,
// z -> +inf gives 1).  The library expf and divide put range-check branches
// around every element of the epilogue.
__device__ __forceinline__ float sigmoid_hw(float z) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504088896341f * z));
}
// 1 / max(|x|, 1e-6) from the sum of squares, as one hardware reciprocal square
// root (sqrt is monotone, so max(sqrt(ss), 1e-6) = sqrt(max(ss, 1e-12)))
__device__ __forceinline__ float inv_norm(float ss) { return __builtin_amdgcn_rsqf(fmaxf(ss, 1e-12f)); }

// Sum over aligned groups of NL = 16 or 32 lanes, result in every lane of the
// group, by register moves only: DPP swaps within quads, mirrored half rows and
// mirrored rows give 16-lane sums; v_permlane16_swap exchanges neighbouring
// rows for 32.  (A shuffle per step would be an LDS round trip each.)
template <int CTRL>
__device__ __forceinline__ float gemm_dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int NL>
__device__ __forceinline__ float lanes_sum(float x) {
    static_assert(NL == 16 || NL == 32, "16- or 32-lane groups");
    x += gemm_dpp<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += gemm_dpp<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += gemm_dpp<0x141>(x);   // row_half_mirror
    x += gemm_dpp<0x140>(x);   // row_mirror
    if constexpr (NL == 32) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    return x;
}

// Element offset of 16-byte segment `seg` of LDS row `r` (64 bf16 per row).
__device__ __forceinline__ int swz(int r, int seg) {
    return r * BK + 8 * (seg ^ (r & 7) ^ ((r >> 3) & 1));
}

// Buffer descriptor over bytes [p, p + n): loads at offsets >= n return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void *p, int n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, n, 0x00020000);
}
// 16 bytes per lane from the buffer at byte offset voff into LDS at dst + 16 lane
// (dst wave-uniform).  A plain function: the builtin must not sit in a generic
// lambda of a kernel template (the host pass would drop the kernel's stub).
__device__ __forceinline__ void gemm_dma16(__amdgpu_buffer_rsrc_t r, uint16_t *dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, 0, 0, 0);
}

// A short tile: SHORT_M rows of the at most 32 columns past N's last multiple
// of 256, which in a projection are the gate-transform columns (beta, alpha).
// Its products are few, so the K-tile pipeline would leave it waiting out one
// memory round trip per K-tile; instead each of the NW waves takes K / NW of
// the depth and issues its fragment loads straight from memory, eight k-steps'
// worth in flight together, and the NW partial 64 x 32 sums meet in LDS (red0
// for waves 0-3, red1 for 4-7, 8 KiB each).  Rows past mlim and columns past N
// load a clamped in-range row and are not stored.
template <int NW>
__device__ __forceinline__ void short_gate_tile(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                                                int lda, int ldb, int K, int m0, int mlim, int n0, int N,
                                                const ProjOut &po, float *red0, float *red1, int wave, int lane) {
    static_assert(SHORT_M == 64, "two 32-row accumulator tiles");
    const int l32 = lane & 31, lh = lane >> 5;
    const int KS = K / (16 * NW);   // k-steps per wave (K is a multiple of 128)
    const int kw = wave * 16 * KS + 8 * lh;
    const uint16_t *a0 = A + (size_t)min(m0 + l32, mlim - 1) * lda + kw;
    const uint16_t *a1 = A + (size_t)min(m0 + 32 + l32, mlim - 1) * lda + kw;
    const uint16_t *b0 = B + (size_t)min(n0 + l32, N - 1) * ldb + kw;
    f32x16 c0 = {}, c1 = {};
    constexpr int KB = 8;
    for (int ks = 0; ks < KS; ks += KB) {
        bf16x8 xa0[KB], xa1[KB], xb[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u)
            if (ks + u < KS) {
                xa0[u] = *reinterpret_cast<const bf16x8 *>(a0 + 16 * (ks + u));
                xa1[u] = *reinterpret_cast<const bf16x8 *>(a1 + 16 * (ks + u));
                xb[u] = *reinterpret_cast<const bf16x8 *>(b0 + 16 * (ks + u));
            }
#pragma unroll
        for (int u = 0; u < KB; ++u)
            if (ks + u < KS) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa0[u], xb[u], c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa1[u], xb[u], c1, 0, 0, 0);
            }
    }
    // register r of tile i holds row 32 i + 8 (r/4) + 4 lh + r%4, column l32
    float *red = (wave < 4 ? red0 : red1) + (wave & 3) * (SHORT_M * 32);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * lh + (r & 3);
        red[row * 32 + l32] = c0[r];
        red[(32 + row) * 32 + l32] = c1[r];
    }
    __syncthreads();
    const int Hd = po.H * po.d, g0 = (po.g ? 4 : 3) * Hd;   // first gate-transform column
    for (int o = wave * 64 + lane; o < SHORT_M * 32; o += 64 * NW) {
        float z = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) z += (w < 4 ? red0 : red1)[(w & 3) * (SHORT_M * 32) + o];
        const int m = m0 + (o >> 5), n = n0 + (o & 31), c = n - g0;
        if (m < mlim && n < N && po.beta && c >= 0 && c < 2 * po.H) {
            if (c < po.H) po.beta[(size_t)m * po.H + c] = sigmoid_hw(z);
            else po.alpha[(size_t)m * po.H + c - po.H] = sigmoid_hw(-z);   // exp(-softplus(z))
        }
    }
}

// NW waves: 4 (wave tiles 128 x 128, one wave per SIMD) or 8 (wave tiles 64 x 128,
// two waves per SIMD, so that one wave's products cover the other's LDS reads)
template <int EPI, int DH, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void gemm_bf16_nt_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int M, int N, int K,
                         int lda, int ldb, ProjOut po, ResidOut ro) {
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    constexpr int WR = 2 * BM / NW;     // rows of a wave tile
    constexpr int NI = WR / 32;         // 32-row accumulator tiles per wave
    constexpr int NCH = 32 / NW;        // 1 KiB DMA chunks per wave per operand and K-tile
    // two buffers as four distinct arrays: the compiler can then tell that the DMA
    // into one buffer does not alias the fragment reads of the other
    __shared__ __attribute__((aligned(1024))) uint16_t A0[BM * BK], A1[BM * BK], B0[BN * BK], B1[BN * BK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lh = lane >> 5;
    const int n_tiles = gemm_full_col_tiles(N);
    const int full = ((M + BM - 1) / BM) * n_tiles;
    int m0, n0, mrows;
    if ((int)blockIdx.x < full) {
        const int logical = xcd_logical(blockIdx.x, full);
        m0 = (logical / n_tiles) * BM;
        n0 = (logical % n_tiles) * BN;
        mrows = min(M - m0, BM);
    } else {   // short tile of the last columns
        m0 = ((int)blockIdx.x - full) * SHORT_M;
        n0 = n_tiles * BN;
        mrows = min(M - m0, SHORT_M);
    }
    const int mlim = m0 + mrows;   // rows past this are zero in LDS and not stored
    if constexpr (EPI == EPI_PROJ) {
        if ((int)blockIdx.x >= full) {
            short_gate_tile<NW>(A, B, lda, ldb, K, m0, mlim, n0, N, po, reinterpret_cast<float *>(A0),
                                reinterpret_cast<float *>(A1), wave, lane);
            return;
        }
    }

    // K-tiles (256 rows x 64 bf16 of A and of B) go from memory straight into LDS
    // by LDS-DMA buffer loads, 16 bytes per lane: wave w fills the 1 KiB chunks
    // w, w + 4, ... (8 rows each); lane i of chunk c writes bytes 16 i of it, i.e.
    // row 8 c + i / 8, physical segment i % 8, and fetches the logical segment the
    // swizzle maps there.  The descriptors end at the tile's last row of A (B) in
    // range, so rows past M (N) read as zero.  K-tile kt + 2 is requested into
    // K-tile kt's buffer at kt's barrier and waited for at kt + 1's, so a tile of
    // products covers the load latency, with no staging registers.
    int voa[NCH], vob[NCH];
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
        const int row = 8 * (wave + NW * n) + (lane >> 3);
        const int lseg = (lane & 7) ^ (row & 7) ^ ((row >> 3) & 1);
        voa[n] = 2 * (row * lda + 8 * lseg);
        vob[n] = 2 * (row * ldb + 8 * lseg);
    }
    const int abytes = 2 * mrows * lda, bbytes = 2 * min(N - n0, BN) * ldb;
    const uint16_t *Ag = A + (size_t)m0 * lda, *Bg = B + (size_t)n0 * ldb;
    auto dma_tile = [&](int kt, auto bufc) {
        uint16_t *Ad = decltype(bufc)::value ? A1 : A0;
        uint16_t *Bd = decltype(bufc)::value ? B1 : B0;
        const int k0 = kt * BK;   // kt may be one past the last tile: empty views, the copies write zeros
        const __amdgpu_buffer_rsrc_t ra = gemm_rsrc(Ag + k0, max(abytes - 2 * k0, 0));
        const __amdgpu_buffer_rsrc_t rb = gemm_rsrc(Bg + k0, max(bbytes - 2 * k0, 0));
#pragma unroll
        for (int n = 0; n < NCH; ++n) {
            gemm_dma16(ra, Ad + 512 * (wave + NW * n), voa[n]);
            gemm_dma16(rb, Bd + 512 * (wave + NW * n), vob[n]);
        }
    };

    f32x16 acc[NI][4];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // fragment reads of k-step ks (K offset 16 ks) of one LDS buffer
    int arow[NI], brow[4];
#pragma unroll
    for (int i = 0; i < NI; ++i) arow[i] = WR * wm + 32 * i + l32;
#pragma unroll
    for (int j = 0; j < 4; ++j) brow[j] = 128 * wn + 32 * j + l32;

    // The K loop for a wave whose first NJ 32-column blocks hold columns in range
    // (4; for the last columns' tiles 1; 0 for a wave with no rows or columns in
    // range): the other blocks' products and the unused fragment reads are left
    // out, the copies and barriers are not.
    auto kloop = [&](auto njc) {
        constexpr int NJ = decltype(njc)::value;
        constexpr int NJB = NJ > 0 ? NJ : 1;
        constexpr int NRJ = NJ > 0 ? NI + NJ : 0;   // fragment reads per k-step
        constexpr int NMJ = NI * NJ;                // products per k-step
        // Fragments by k-step parity.  A K-tile's k-steps 0..2 run with the reads
        // of k-steps 1..3; then this wave waits for the next K-tile's DMA, the
        // workgroup meets (every read of this tile's buffer is done, so the DMA
        // two K-tiles ahead can go into it), and k-step 3 runs with the reads of
        // the next tile's k-step 0, so no tile starts on an LDS round trip.
        bf16x8 fa[2][NI], fb[2][NJB];
        auto frags = [&](auto bufc, int ks, bf16x8 *xa, bf16x8 *xb) {
            if constexpr (NJ > 0) {
                const uint16_t *As = decltype(bufc)::value ? A1 : A0;
                const uint16_t *Bs = decltype(bufc)::value ? B1 : B0;
                const int seg = 2 * ks + lh;
#pragma unroll
                for (int i = 0; i < NI; ++i) xa[i] = *reinterpret_cast<const bf16x8 *>(&As[swz(arow[i], seg)]);
#pragma unroll
                for (int j = 0; j < NJ; ++j) xb[j] = *reinterpret_cast<const bf16x8 *>(&Bs[swz(brow[j], seg)]);
            }
        };
        auto mul = [&](const bf16x8 *xa, const bf16x8 *xb) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], xb[j], acc[i][j], 0, 0, 0);
        };
        // the k-step's products; the fragment reads issued just before go out one per product
        auto products = [&](const bf16x8 *xa, const bf16x8 *xb) {
            mul(xa, xb);
            if constexpr (NJ == 4) {
#pragma unroll
                for (int n = 0; n < NRJ; ++n) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NMJ - NRJ, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        auto head = [&](auto bufc) {   // k-steps 0 .. 2 of the tile in bufc
#pragma unroll
            for (int ks = 0; ks < BK / 16 - 1; ++ks) {
                frags(bufc, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
                products(fa[ks & 1], fb[ks & 1]);
            }
        };
        // k-step 3, with k-step 0 of the tile in nextc and the copies of K-tile kn
        // into buffer dmac (empty views past the last tile), one copy per product
        // so that the copies' issue time overlaps the matrix pipe
        auto tail = [&](auto nextc, int kn, auto dmac) {
            static_assert(BK / 16 == 4, "k-step 3 uses the odd fragment set");
            frags(nextc, 0, fa[0], fb[0]);
            dma_tile(kn, dmac);
            mul(fa[1], fb[1]);
            if constexpr (NJ == 4) {
                static_assert(2 * NCH == NMJ, "one copy per product");
#pragma unroll
                for (int n = 0; n < NRJ; ++n) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
#pragma unroll
                for (int n = 0; n < NMJ - NRJ; ++n) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };

        // K is a multiple of 128 (the looped drivers require d_model and H*d to be),
        // so the K-tiles come in pairs, one per buffer
        const int KT = K / BK;
        const std::integral_constant<int, 0> c0{};
        const std::integral_constant<int, 1> c1{};
        dma_tile(0, c0);
        dma_tile(1, c1);
        wait_vmem_all();
        __syncthreads();
        frags(c0, 0, fa[0], fb[0]);
        for (int kt = 0; kt < KT; kt += 2) {
            head(c0);                         // K-tile kt
            wait_vmem_all();                  // K-tile kt + 1 (buffer 1) has landed
            __syncthreads();
            tail(c1, min(kt + 2, KT), c0);    // K-tile kt + 2 into buffer 0
            head(c1);                         // K-tile kt + 1
            wait_vmem_all();                  // K-tile kt + 2 (buffer 0) has landed
            __syncthreads();
            tail(c0, min(kt + 3, KT), c1);    // past the last tile its reads are stale and unused
        }
        wait_vmem_all();   // the empty copies past the last tile have landed
        __syncthreads();   // the epilogue stages through the K-tile buffers
    };
    // columns and rows of this wave in range (wave-uniform)
    const int wcols = N - n0 - 128 * wn, wrows = mlim - m0 - WR * wm;
    if (wrows > 0 && wcols > 32) kloop(std::integral_constant<int, 4>{});
    else if (wrows > 0 && wcols > 0) kloop(std::integral_constant<int, 1>{});
    else kloop(std::integral_constant<int, 0>{});

    // ---- epilogue: register r of tile (i, j) holds
    //      C[m0 + WR wm + 32 i + 8 (r/4) + 4 lh + r%4][n0 + 128 wn + 32 j + l32] ----
    // Blocks of SR rows of the wave's tile go through LDS, in the K-tile buffers,
    // idle since the loop's last barrier: with four waves each wave has a buffer
    // of its own and stages 32 rows, with eight two waves share one, 16 rows each.
    constexpr int SR = NW == 4 ? 32 : 16;
    constexpr int RP = 132;   // fp32 pitch of a staged row (16-byte rows, no 2-way conflict)
    static_assert((NW / 4) * SR * RP * 4 <= BM * BK * 2, "staging fits a K-tile buffer");
    const int sb = NW == 4 ? wave : wave >> 1;
    float *stage = reinterpret_cast<float *>(sb == 0 ? A0 : (sb == 1 ? A1 : (sb == 2 ? B0 : B1))) +
                   (NW == 4 ? 0 : (wave & 1) * SR * RP);
    // rows [SR h, SR h + SR) of accumulator tile i into the stage: registers r of
    // that block are SR/2 h .. SR/2 h + SR/2 - 1
    auto stage_block = [&](int i, int h) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < SR / 2; ++r) {
                const int rr = (SR / 2) * h + r;
                stage[(8 * (rr >> 2) + 4 * lh + (rr & 3) - SR * h) * RP + 32 * j + l32] = acc[i][j][rr];
            }
    };
    const int nw = n0 + 128 * wn;   // first column of this wave
    if constexpr (EPI == EPI_PROJ) {
        const int Hd = po.H * po.d;
        const int NRB = po.g ? 4 : 3;               // head-width column blocks before the gates
        if (nw < NRB * Hd) {
            // q, k, v or g columns; the wave's 128 columns hold whole heads (Hd % 128 == 0).
            // A half-wave holds a staged row, 4 columns per lane, so the per-head L2
            // norm is a reduction over the head's DH / 4 lanes and each lane stores
            // 8 bytes.
            const int region = nw / Hd;             // 0 q, 1 k, 2 v, 3 g
            uint16_t *dst = region == 0 ? po.q : (region == 1 ? po.k : (region == 2 ? po.v : po.g));
            const int c0 = nw - region * Hd + 4 * l32;
            const bool norm = region < 2 && po.norm;
            // one straight-line pass per transform (0 none, 1 L2 norm, 2 sigmoid),
            // the choice made once per wave
            auto blocks = [&](auto modec) {
                constexpr int MODE = decltype(modec)::value;
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int h = 0; h < 32 / SR; ++h) {
                        stage_block(i, h);
                        const int mb = m0 + WR * wm + 32 * i + SR * h + lh;   // row of piece q is mb + 2 q
#pragma unroll
                        for (int q = 0; q < SR / 2; ++q) {
                            const float4 c = *reinterpret_cast<const float4 *>(&stage[(2 * q + lh) * RP + 4 * l32]);
                            float x[4] = {c.x, c.y, c.z, c.w};
                            if constexpr (MODE == 1) {
                                const float ss =
                                    lanes_sum<DH / 4>(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
                                const float sc = inv_norm(ss);
#pragma unroll
                                for (int e = 0; e < 4; ++e) x[e] *= sc;
                            } else if constexpr (MODE == 2) {
#pragma unroll
                                for (int e = 0; e < 4; ++e) x[e] = sigmoid_hw(x[e]);
                            }
                            const int m = mb + 2 * q;
                            if (m < mlim) {
                                uint2 u;
                                u.x = (uint32_t)bf16_bits(x[0]) | ((uint32_t)bf16_bits(x[1]) << 16);
                                u.y = (uint32_t)bf16_bits(x[2]) | ((uint32_t)bf16_bits(x[3]) << 16);
                                *reinterpret_cast<uint2 *>(&dst[(size_t)m * Hd + c0]) = u;
                            }
                        }
                    }
            };
            if (norm) blocks(std::integral_constant<int, 1>{});
            else if (region == 3) blocks(std::integral_constant<int, 2>{});
            else blocks(std::integral_constant<int, 0>{});
        } else {
            // gate columns: beta (first H) and alpha (next H)
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = nw + 32 * j + l32 - NRB * Hd;
                    if (!po.beta || c >= 2 * po.H) continue;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = m0 + WR * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                        if (m >= mlim) continue;
                        const float z = acc[i][j][r];
                        if (c < po.H) po.beta[(size_t)m * po.H + c] = sigmoid_hw(z);
                        else po.alpha[(size_t)m * po.H + c - po.H] = sigmoid_hw(-z);  // exp(-softplus(z))
                    }
                }
        }
    } else {
        // Residual update, one staged block at a time, so that h is read and
        // written as whole 512-byte row pieces, all loads of a block in flight
        // together.  N is a multiple of 128, so a wave's columns are all in range
        // or all out.
        if (nw >= N) return;
        const int n = nw + 4 * l32;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int h = 0; h < 32 / SR; ++h) {
                stage_block(i, h);
                const int mb = m0 + WR * wm + 32 * i + SR * h + lh;   // row of piece q is mb + 2 q
                float4 hv[SR / 2];
#pragma unroll
                for (int q = 0; q < SR / 2; ++q) {
                    const int m = min(mb + 2 * q, mlim - 1);   // rows past the tile's load its last, store nothing
                    hv[q] = *reinterpret_cast<const float4 *>(&ro.h[(size_t)m * N + n]);
                }
#pragma unroll
                for (int q = 0; q < SR / 2; ++q) {
                    const float4 c = *reinterpret_cast<const float4 *>(&stage[(2 * q + lh) * RP + 4 * l32]);
                    const float4 hn = make_float4(hv[q].x + c.x, hv[q].y + c.y, hv[q].z + c.z, hv[q].w + c.w);
                    const int m = mb + 2 * q;
                    if (m < mlim) {
                        const size_t o = (size_t)m * N + n;
                        *reinterpret_cast<float4 *>(&ro.h[o]) = hn;
                        uint2 u;
                        u.x = (uint32_t)bf16_bits(hn.x) | ((uint32_t)bf16_bits(hn.y) << 16);
                        u.y = (uint32_t)bf16_bits(hn.z) | ((uint32_t)bf16_bits(hn.w) << 16);
                        *reinterpret_cast<uint2 *>(&ro.xb[o]) = u;
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Small-M variant (the decode chain's M = batch of sequences): 64 x 128 tiles
// so that a few hundred rows still give ~200 workgroups.  Four waves, wave w
// owning columns 32w .. 32w+31 of the tile for all 64 rows (two 32x32 MFMA
// accumulators).  With M this small the products are cheap and the kernel
// streams B: K-tiles of 64 go from memory into LDS by LDS-DMA buffer loads
// through five stages (swizzled as in the large kernel), four K-tiles in flight
// per workgroup.  Each stage is its own pair of __shared__ arrays, selected at
// compile time (the K loop is unrolled by the stage count), so that the
// compiler can tell a DMA into one stage from the fragment reads of another.
// The accumulators then go to LDS and the epilogue works row by row: four
// threads per row, 32 columns each, so the per-head L2 norm is a two-step
// shuffle reduction and every global access is a 16-byte vector.  The residual
// product also has a 32-row form (one accumulator per wave, eight threads per
// row in the epilogue) for shapes with too few 64-row tiles to fill the GPU.
constexpr int SBN = 128, SNS = 5;   // columns, LDS stages

// Logical index of block `bid` of `n` such that each XCD (the hardware deals
// blocks round-robin, block b to XCD b % 8) holds one contiguous run of logical
// indices, for any n: XCD x takes n / 8 blocks, one more when x < n % 8.
__device__ __forceinline__ int xcd_run(int bid, int n) {
    const int q = n >> 3, r = n & 7, x = bid & 7;
    return x * q + min(x, r) + (bid >> 3);
}

// SBM: tile rows (64; 32 for the residual product only); KTC: K-tiles known at
// compile time (0: K at run time)
template <int EPI, int DH, int KTC, int SBM = 64>
__global__ __launch_bounds__(256) void gemm_small_kernel(const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ B, int M, int N, int K,
                                                         ProjOut po, ResidOut ro) {
    static_assert(SBM == 64 || (SBM == 32 && EPI == EPI_RESID), "tile rows");
    constexpr int A_EL = SBM * BK, B_EL = SBN * BK, CP = SBN + 4;
    constexpr int NA = SBM / 32;   // A chunks per wave, accumulators per wave
    // 1 KiB DMA chunks per stage: A SBM / 8, B 16; wave w takes A chunks w + 4 j and B chunks w + 4 j
    constexpr int DMA_PER_WAVE = NA + 4;
    // one array per stage (A tile, then B tile): the compiler tracks only a few
    // distinct LDS-DMA targets, and ten would make every fragment read wait for
    // every DMA in flight
    __shared__ __attribute__((aligned(1024))) uint16_t S0[A_EL + B_EL], S1[A_EL + B_EL], S2[A_EL + B_EL],
        S3[A_EL + B_EL], S4[A_EL + B_EL];
    __shared__ __attribute__((aligned(16))) float Cs[SBM * CP];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    // the row tiles sharing a weight panel are consecutive logical tiles, so
    // one XCD's L2 fetches each panel once
    const int m_tiles = (M + SBM - 1) / SBM;
    const int logical = xcd_run(blockIdx.x, gridDim.x);
    const int mt = logical % m_tiles, nt = logical / m_tiles;
    const int m0 = mt * SBM, n0 = nt * SBN;

    // lane i of a chunk writes bytes 16 i of it: row 8 c + i / 8, physical
    // segment i % 8, holding the logical segment the swizzle maps there
    int voa[NA], vob[4];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int row = 8 * (wave + 4 * j) + (lane >> 3);
        voa[j] = 2 * (row * K + 8 * ((lane & 7) ^ (row & 7) ^ ((row >> 3) & 1)));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 8 * (wave + 4 * j) + (lane >> 3);
        vob[j] = 2 * (row * K + 8 * ((lane & 7) ^ (row & 7) ^ ((row >> 3) & 1)));
    }
    // descriptors end at the tile's last row in range: rows past M (N) read zero
    const int abytes = 2 * min(M - m0, SBM) * K, bbytes = 2 * min(N - n0, SBN) * K;
    const uint16_t *Ag = A + (size_t)m0 * K, *Bg = B + (size_t)n0 * K;
    auto dma = [&](int kt, uint16_t *Ad, uint16_t *Bd) {
        const int k0 = kt * BK;
        const __amdgpu_buffer_rsrc_t ra = gemm_rsrc(Ag + k0, abytes - 2 * k0);
        const __amdgpu_buffer_rsrc_t rb = gemm_rsrc(Bg + k0, bbytes - 2 * k0);
#pragma unroll
        for (int j = 0; j < NA; ++j) gemm_dma16(ra, Ad + 512 * (wave + 4 * j), voa[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) gemm_dma16(rb, Bd + 512 * (wave + 4 * j), vob[j]);
    };
    f32x16 acc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) acc[i] = f32x16{};
    auto compute = [&](const uint16_t *As, const uint16_t *Bs) {
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int seg = 2 * ks + lh;
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(&Bs[swz(32 * wave + l32, seg)]);
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&As[swz(32 * i + l32, seg)]);
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
            }
        }
    };
    // K-tile kt sits in stage kt % SNS.  Step kt: wait for this wave's DMAs of
    // K-tile kt (those of the SNS - 2 later K-tiles may still be in flight),
    // barrier (every wave's share has landed, and every wave has finished
    // reading the stage that K-tile kt + SNS - 1 is about to overwrite), issue
    // that K-tile, multiply K-tile kt.
    // With the K-tile count known at compile time the K loop unrolls completely;
    // the compiler's wait counts are then exact and the DMAs of the later
    // stages stay in flight while a stage is read (in a loop they are merged at
    // the back-edge into a wait for all but the newest stage).
    const int KT = KTC > 0 ? KTC : K / BK;
    // stage arrays by compile-time index (so each access names its own array)
    auto stA = [&](auto sc) -> uint16_t * {
        constexpr int S = decltype(sc)::value;
        if constexpr (S == 0) return S0; else if constexpr (S == 1) return S1;
        else if constexpr (S == 2) return S2; else if constexpr (S == 3) return S3; else return S4;
    };
    auto stB = [&](auto sc) -> uint16_t * { return stA(sc) + A_EL; };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // every step issues one K-tile (past the last, the last again, into the
    // stage being retired, which is never read again), so the DMAs in flight
    // behind K-tile kt are always SNS - 2 K-tiles' worth and the wait is constant
    dma(0, stA(I0{}), stB(I0{}));
    dma(min(1, KT - 1), stA(I1{}), stB(I1{}));
    dma(min(2, KT - 1), stA(I2{}), stB(I2{}));
    dma(min(3, KT - 1), stA(I3{}), stB(I3{}));
    auto step = [&](int kt, auto sc) {
        constexpr int S = decltype(sc)::value, SN = (S + SNS - 1) % SNS;
        const std::integral_constant<int, S> cs{};
        const std::integral_constant<int, SN> cn{};
        wait_vmem_le<(SNS - 2) * DMA_PER_WAVE>();
        // A bare hardware barrier: __syncthreads (a release fence, which counts
        // the LDS-DMA writes still in flight) would wait for every later
        // K-tile too.  What it would order is covered otherwise: this wave's
        // share of K-tile kt has landed (the wait above), and every fragment
        // read of the stage about to be overwritten was consumed by the
        // previous step's products before this wave reached the barrier.
        __builtin_amdgcn_s_barrier();
        dma(min(kt + SNS - 1, KT - 1), stA(cn), stB(cn));
        __builtin_amdgcn_sched_barrier(0);
        compute(stA(cs), stB(cs));
    };
    static_assert(SNS == 5, "the step sequence below names five stages");
    auto five = [&](int kt) {
        step(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < KT) step(kt + 1, std::integral_constant<int, 1>{});
        if (kt + 2 < KT) step(kt + 2, std::integral_constant<int, 2>{});
        if (kt + 3 < KT) step(kt + 3, std::integral_constant<int, 3>{});
        if (kt + 4 < KT) step(kt + 4, std::integral_constant<int, 4>{});
    };
    if constexpr (KTC > 0) {
#pragma unroll
        for (int kt = 0; kt < KTC; kt += SNS) five(kt);
    } else {
        for (int kt = 0; kt < KT; kt += SNS) five(kt);
    }

    // accumulators -> LDS: register r of tile i holds row 32 i + 8 (r/4) + 4 lh + r%4,
    // column 32 wave + l32
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) Cs[(32 * i + 8 * (r >> 2) + 4 * lh + (r & 3)) * CP + 32 * wave + l32] = acc[i][r];
    __syncthreads();

    // epilogue: thread (row, part): TPR = 256 / SBM threads per row, each CPT
    // columns (64 rows: four threads of 32 columns)
    constexpr int TPR = 256 / SBM, CPT = SBN / TPR;
    const int row = tid / TPR, q4 = tid % TPR;
    const int m = m0 + row;
    const int c0 = CPT * q4;
    const float *cr = Cs + row * CP + c0;
    if constexpr (EPI == EPI_RESID) {
        if (m < M) {
#pragma unroll
            for (int j = 0; j < CPT; j += 8) {
                const int n = n0 + c0 + j;
                if (n >= N) break;
                float *hp = ro.h + (size_t)m * N + n;
                float4 h0 = *reinterpret_cast<float4 *>(hp), h1 = *reinterpret_cast<float4 *>(hp + 4);
                h0.x += cr[j + 0]; h0.y += cr[j + 1]; h0.z += cr[j + 2]; h0.w += cr[j + 3];
                h1.x += cr[j + 4]; h1.y += cr[j + 5]; h1.z += cr[j + 6]; h1.w += cr[j + 7];
                *reinterpret_cast<float4 *>(hp) = h0;
                *reinterpret_cast<float4 *>(hp + 4) = h1;
                u32x4 xb;
                xb[0] = (uint32_t)bf16_bits(h0.x) | ((uint32_t)bf16_bits(h0.y) << 16);
                xb[1] = (uint32_t)bf16_bits(h0.z) | ((uint32_t)bf16_bits(h0.w) << 16);
                xb[2] = (uint32_t)bf16_bits(h1.x) | ((uint32_t)bf16_bits(h1.y) << 16);
                xb[3] = (uint32_t)bf16_bits(h1.z) | ((uint32_t)bf16_bits(h1.w) << 16);
                *reinterpret_cast<u32x4 *>(ro.xb + (size_t)m * N + n) = xb;
            }
        }
    } else {
        const int Hd = po.H * po.d;
        const int NR = po.g ? 4 : 3;
        if (n0 < NR * Hd) {
            // the tile lies in one region (Hd is a multiple of 128); heads of DH columns
            const int region = n0 / Hd;
            uint16_t *dst = region == 0 ? po.q : (region == 1 ? po.k : (region == 2 ? po.v : po.g));
            float scale = 1.f;
            if (region < 2 && po.norm) {
                float ss = 0.f;
#pragma unroll
                for (int j = 0; j < 32; ++j) ss += cr[j] * cr[j];
                ss += __shfl_xor(ss, 1);                      // 64 columns
                if constexpr (DH == 128) ss += __shfl_xor(ss, 2);   // 128 columns
                scale = inv_norm(ss);
            }
            if (m < M) {
                const int c = n0 - region * Hd + c0;
#pragma unroll
                for (int j = 0; j < 32; j += 8) {
                    u32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x0 = cr[j + 2 * e] * scale, x1 = cr[j + 2 * e + 1] * scale;
                        if (region == 3) {
                            x0 = sigmoid_hw(x0);
                            x1 = sigmoid_hw(x1);
                        }
                        o[e] = (uint32_t)bf16_bits(x0) | ((uint32_t)bf16_bits(x1) << 16);
                    }
                    *reinterpret_cast<u32x4 *>(dst + (size_t)m * Hd + c + j) = o;
                }
            }
        } else if (po.beta && m < M) {
            // gate columns: beta (first H) and alpha (next H)
            for (int j = 0; j < 32; ++j) {
                const int c = n0 + c0 + j - NR * Hd;
                if (c >= 2 * po.H) break;
                const float z = cr[j];
                if (c < po.H) po.beta[(size_t)m * po.H + c] = sigmoid_hw(z);
                else po.alpha[(size_t)m * po.H + c - po.H] = sigmoid_hw(-z);
            }
        }
    }
}

// The 256 x 256 kernel unless it would launch fewer than 64 workgroups.
bool use_small(int M, int N) { return (long)((M + BM - 1) / BM) * ((N + BN - 1) / BN) < 64; }

}  // namespace

hipError_t launch_gemm_proj(const uint16_t *X, const uint16_t *W, int M, int N, int K, uint16_t *q, uint16_t *k,
                            uint16_t *v, uint16_t *g, float *beta, float *alpha, int H, int d, hipStream_t s,
                            bool norm_qk) {
    if (K <= 0 || K % (2 * BK) != 0) return hipErrorInvalidValue;   // K-tiles are consumed in pairs
    ProjOut po{q, k, v, g, beta, alpha, H, d, norm_qk ? 1 : 0};
    ResidOut ro{nullptr, nullptr};
    if (use_small(M, N)) {
        const unsigned sg = (unsigned)((M + 63) / 64) * (unsigned)((N + SBN - 1) / SBN);
        if (d == 64)
            hipLaunchKernelGGL((gemm_small_kernel<EPI_PROJ, 64, 0>), dim3(sg), dim3(256), 0, s, X, W, M, N, K, po, ro);
        else
            if (K == 32 * BK)
                hipLaunchKernelGGL((gemm_small_kernel<EPI_PROJ, 128, 32>), dim3(sg), dim3(256), 0, s, X, W, M, N, K, po,
                                   ro);
            else
                hipLaunchKernelGGL((gemm_small_kernel<EPI_PROJ, 128, 0>), dim3(sg), dim3(256), 0, s, X, W, M, N, K, po,
                                   ro);
        return hipGetLastError();
    }
    const unsigned grid = gemm_grid(M, N);
    if (d == 64)
        hipLaunchKernelGGL((gemm_bf16_nt_kernel<EPI_PROJ, 64, GEMM_NW>), dim3(grid), dim3(64 * GEMM_NW), 0, s, X, W, M, N, K, K, K, po, ro);
    else
        hipLaunchKernelGGL((gemm_bf16_nt_kernel<EPI_PROJ, 128, GEMM_NW>), dim3(grid), dim3(64 * GEMM_NW), 0, s, X, W, M, N, K, K, K, po, ro);
    return hipGetLastError();
}

hipError_t launch_gemm_resid(const uint16_t *O, const uint16_t *W, int M, int N, int K, float *h, uint16_t *xb,
                             hipStream_t s) {
    if (K <= 0 || K % (2 * BK) != 0 || N % 128 != 0) return hipErrorInvalidValue;
    ProjOut po{};
    ResidOut ro{h, xb};
    if (use_small(M, N)) {
        const unsigned sg = (unsigned)((M + 63) / 64) * (unsigned)((N + SBN - 1) / SBN);
        const unsigned sg32 = (unsigned)((M + 31) / 32) * (unsigned)((N + SBN - 1) / SBN);
        if (K == 32 * BK && 2 * sg < (unsigned)device_cus())   // few 64-row tiles: 32-row tiles, twice as many
            hipLaunchKernelGGL((gemm_small_kernel<EPI_RESID, 128, 32, 32>), dim3(sg32), dim3(256), 0, s, O, W, M, N, K,
                               po, ro);
        else if (K == 32 * BK)
            hipLaunchKernelGGL((gemm_small_kernel<EPI_RESID, 128, 32>), dim3(sg), dim3(256), 0, s, O, W, M, N, K, po, ro);
        else
            hipLaunchKernelGGL((gemm_small_kernel<EPI_RESID, 128, 0>), dim3(sg), dim3(256), 0, s, O, W, M, N, K, po, ro);
        return hipGetLastError();
    }
    const unsigned grid = gemm_grid(M, N);
    hipLaunchKernelGGL((gemm_bf16_nt_kernel<EPI_RESID, 128, GEMM_NW>), dim3(grid), dim3(64 * GEMM_NW), 0, s, O, W, M, N, K, K, K, po, ro);
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
