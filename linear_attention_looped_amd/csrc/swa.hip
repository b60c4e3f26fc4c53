// swa.hip -- causal sliding-window softmax attention, the sparse LT2 mixer
// (LT2 explainer, paithon.it, section "Sostituire il motore": each token attends
// to a window of the w most recent positions, itself included):
//
//   o_t = sum_{j = max(0, t-w+1)}^{t} softmax_j(q_t . k_j / sqrt(d)) v_j
//
// per (batch, head), q, k, v bf16 [B, L, H, d], o bf16 or fp32.
//
// One workgroup = one (b, h) and 128 consecutive queries; four waves of 32
// queries each.  Keys and values stream through LDS in tiles of 64 tokens,
// double-buffered: the next tile is loaded straight into the other LDS buffer
// (buffer loads with the LDS-DMA bit, 16 bytes per lane, no staging registers)
// while the current one is used, so one barrier per tile suffices.
//
// Per wave and tile the scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: the A operand is a K row fragment read from LDS,
// the B operand the wave's Q fragments, held in registers for the whole kernel.
// In the accumulator layout (register r of lane l holds row 8(r/4) + 4(l/32) +
// r%4, column l%32) every lane then owns ONE query (column l%32) and 16 of each
// 32 keys, so the online softmax is in-lane apart from one exchange with the
// other half-wave.  The output is accumulated transposed as well, O^T += V^T P^T:
// the probabilities already sit in the B-operand layout once the key order of
// the contraction is permuted to match the accumulator rows (lane half h, slot
// s <-> key 8(s/4) + 4h + s%4 of each 16-key step), and the V^T A operand comes
// from the row-major V tile through LDS transpose reads with the same key order.
//
// Softmax in base 2: scores are scaled by log2(e)/sqrt(d) and exponentiated
// with exp2; the running maximum starts at a large finite negative value so a
// fully masked tile contributes exp2(-inf) = 0 without producing NaN.  The
// accumulated output is rescaled only when some lane's maximum has grown by
// more than 8 (a factor 256): otherwise the stale maximum is kept, which bounds
// the probabilities by 256 -- harmless in bf16 and fp32 -- and skips the
// rescale on most tiles.  Masking is applied only on tiles that cross the
// causal diagonal or the window's start; tiles wholly outside a wave's range
// are skipped by that wave.
//
// K and V tiles are read through buffer descriptors whose range ends at the
// sequence's last token, so rows past the end read as zero (and are masked)
// without clamping, and each thread's offset inside a tile stays constant.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace lt2 {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((address_space(3))) short4_t lds_short4;

constexpr int SWA_QT = 128;   // queries per workgroup
constexpr int SWA_KT = 64;    // keys per LDS tile
constexpr int SWA_NTH = 256;  // four waves

// max (or sum) of a value over lanes l and l ^ 32
__device__ __forceinline__ float halves_max(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Buffer descriptor over bytes [p, p + n): loads at offsets >= n return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, n, 0x00020000);
}

// 16 bytes per lane from the buffer at byte offset voff into LDS at dst + 16 lane
// (dst wave-uniform).  Kept out of the kernel's generic lambdas: instantiated
// there by the host pass, the builtin would invalidate the kernel template.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint16_t *dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, 0, 0, 0);
}

template <typename TO>
__device__ __forceinline__ void store4(TO *p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t *p, float a, float b, float c, float d) {
    uint2 u;
    u.x = (uint32_t)bf16_bits(a) | ((uint32_t)bf16_bits(b) << 16);
    u.y = (uint32_t)bf16_bits(c) | ((uint32_t)bf16_bits(d) << 16);
    *reinterpret_cast<uint2 *>(p) = u;
}
template <>
__device__ __forceinline__ void store4<float>(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

// LDS tiles hold 64 rows of d bf16 without padding; the 16-byte segment sigma
// of row r sits at segment sigma ^ swz(r), which keeps both the 16-row fragment
// reads of K and the 4-row transpose reads of V free of bank conflicts.
template <int SPR>
__device__ __forceinline__ int swz(int r) {
    return (4 * (r & 3) + ((r >> 2) & 3)) & (SPR - 1);
}

template <int D, typename TO>
__global__ __launch_bounds__(SWA_NTH) __attribute__((amdgpu_waves_per_eu(2, 2)))
void swa_fwd_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                    TO *__restrict__ out, const uint16_t *__restrict__ gate, int L, int H, int window, int nqt,
                    float sl2) {
    constexpr int KT = SWA_KT;
    constexpr int SPR = D / 8;         // 16-byte segments per row
    constexpr int RPC = 64 / SPR;      // rows per 1 KiB chunk (one wave's LDS-DMA load)
    constexpr int CPW = KT / RPC / 4;  // chunks per wave per tile
    constexpr int TILE = KT * D;       // bf16 per tile
    constexpr int NKS = D / 16;        // k-steps of the score product
    constexpr int NDT = D / 32;        // 32-wide value tiles
    // four distinct arrays (not one [2][...] array): the compiler then knows that
    // a DMA into one buffer does not alias reads of the other, and does not make
    // those reads wait for the DMA
    __shared__ __attribute__((aligned(1024))) uint16_t K0[TILE], K1[TILE], V0[TILE], V1[TILE];

    const int lid = xcd_logical(blockIdx.x, gridDim.x);
    const int qt = lid % nqt;
    const int bh = lid / nqt;
    const int h = bh % H, b = bh / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const size_t tok = (size_t)H * D;                     // elements between consecutive tokens
    const size_t base = ((size_t)b * L * H + h) * D;      // token 0 of this (b, h)
    const int t0 = qt * SWA_QT;
    const int qa = t0 + 32 * wave;                         // first query of this wave
    const int qlast = min(qa + 31, L - 1);
    const bool wave_live = qa < L;
    const int tq = min(qa + l32, L - 1);                   // this lane's query (clamped for the tail)
    const int kbeg = max(0, t0 - window + 1);
    const int kend = min(L, t0 + SWA_QT);                  // exclusive
    const int kt0 = kbeg / KT, kt1 = (kend - 1) / KT;

    // LDS-DMA roles: chunk wave + 4 n of a tile is 1 KiB of LDS; lane i fills its
    // bytes 16 i .. 16 i + 15, i.e. row RPC c + i / SPR, physical segment i % SPR,
    // from the global segment that the swizzle maps there
    int voff[CPW];
#pragma unroll
    for (int n = 0; n < CPW; ++n) {
        const int row = RPC * (wave + 4 * n) + lane / SPR;
        const int sg = (lane % SPR) ^ swz<SPR>(row);
        voff[n] = 2 * (row * (int)tok + 8 * sg);
    }
    auto fetch = [&](int kt, auto bufc) {
        uint16_t *Kd = decltype(bufc)::value ? K1 : K0;
        uint16_t *Vd = decltype(bufc)::value ? V1 : V0;
        // bytes from the tile's first row to the end of the sequence's last row
        const int n = 2 * ((L - 1 - kt * KT) * (int)tok + D);
        const size_t t0b = base + (size_t)kt * KT * tok;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + t0b, n), vr = make_rsrc(v + t0b, n);
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int ch = 512 * (wave + 4 * c);
            dma16(kr, &Kd[ch], voff[c]);
            dma16(vr, &Vd[ch], voff[c]);
        }
    };

    // Q^T fragments: B operand of S^T = K Q^T, query l32, channels 16 ks + 8 hh .. + 7
    bf16x8 qf[NKS];
    {
        const uint16_t *qp = q + base + (size_t)tq * tok + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
    }
    fetch(kt0, std::integral_constant<int, 0>{});
    // the Q fragments must have landed before the tile loop: left to itself the
    // compiler sinks their loads into the loop preheader, and the loop's static
    // wait counts then also hold every tile's MFMAs on that tile's prefetch
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(qf[ks]));

    // per-lane LDS element offsets: K fragment (row l32, channels 16 ks + 8 hh) and
    // the V^T transpose reads (rows 4 hh + e (+ 8), channels 32 dt + 16 (g&1) + 4 c)
    int koff[NKS], vo[2][NDT];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) koff[ks] = l32 * D + 8 * ((2 * ks + hh) ^ swz<SPR>(l32));
    {
        const int e = (lane & 15) >> 2, c4 = lane & 3, g1 = (lane >> 4) & 1;
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int row = 4 * hh + e + 8 * hi;
                const int sg = 4 * dt + 2 * g1 + (c4 >> 1);
                vo[hi][dt] = row * D + 8 * (sg ^ swz<SPR>(row)) + 4 * (c4 & 1);
            }
    }

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m = -1e30f, lsum = 0.f;

    wait_vmem_all();
    __syncthreads();

    auto tile = [&](int kt, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const uint16_t *Kb = buf ? K1 : K0;
        const uint16_t *Vb = buf ? V1 : V0;
        if (kt < kt1) fetch(kt + 1, std::integral_constant<int, buf ^ 1>{});
        const int ka = kt * KT;
        const bool active = wave_live && ka <= qlast && ka + KT - 1 >= qa - window + 1;
        if (active) {
            __builtin_amdgcn_s_setprio(1);
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
            // K fragments two k-steps (eight reads) ahead of their products, so that LDS
            // latency hides behind four MFMAs; the order is pinned by group barriers
            bf16x8 kf[NKS][2];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    kf[ks][kb] = *reinterpret_cast<const bf16x8 *>(&Kb[32 * kb * D + koff[ks]]);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks][kb], qf[ks], s[kb], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);          // k-steps 0, 1
#pragma unroll
            for (int p2 = 0; p2 < NKS / 2; ++p2) {
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);      // products of step pair p2
                if (p2 + 2 < NKS / 2)
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // reads of pair p2 + 2
            }
            // keys outside a query's window: only on tiles that cross the diagonal
            // or the window's start for some live query of the wave
            if (!(ka + KT - 1 <= qa && ka >= qlast - window + 1)) {
                const int jd = ka + 4 * hh - tq;          // key - query of register 0
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int dj = jd + 32 * kb + 8 * (r >> 2) + (r & 3);
                        s[kb][r] = (dj > 0 || dj <= -window) ? -INFINITY : s[kb][r];
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            const float mnew = fmaxf(m, halves_max(mx) * sl2);
            if (__builtin_amdgcn_ballot_w64(mnew > m + 8.f)) {
                const float f = __builtin_amdgcn_exp2f(m - mnew);
                m = mnew;
                lsum *= f;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[dt][r] *= f;
            }
            // probabilities as the B operand of O^T += V^T P^T: 16-key step (kb, half)
            // takes registers 8 half .. 8 half + 7 of s[kb]
            bf16x8 pf[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + e], sl2, -m));
                        lsum += p;
                        pf[kb][hf][e] = (__bf16)p;
                    }
            // V^T fragments of 16-key step st = 2 kb + hf (keys 32 kb + 16 hf + 4 hh + 0..3
            // in slots 0-3, + 8 in slots 4-7), read two steps ahead of their products
            bf16x8 vf[4][NDT];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const uint16_t *vb = &Vb[16 * st * D];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const short4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(vb + vo[0][dt]));
                    const short4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(vb + vo[1][dt]));
                    vf[st][dt] = __builtin_bit_cast(
                        bf16x8, (__attribute__((ext_vector_type(8))) short){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0],
                                                                            hi4[1], hi4[2], hi4[3]});
                }
            }
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st][dt], pf[st >> 1][st & 1], oacc[dt],
                                                                       0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * NDT, 0);    // steps 0, 1
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                __builtin_amdgcn_sched_group_barrier(0x008, NDT, 0);    // products of step st
                if (st + 2 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2 * NDT, 0);   // reads of st + 2
            }
            __builtin_amdgcn_s_setprio(0);
        }
        wait_vmem_all();
        __syncthreads();
    };
    for (int kt = kt0; kt <= kt1; kt += 2) {
        tile(kt, std::integral_constant<int, 0>{});
        if (kt + 1 <= kt1) tile(kt + 1, std::integral_constant<int, 1>{});
    }

    if (!wave_live) return;
    const float lt = halves_sum(lsum);
    const int t = qa + l32;
    if (t >= L) return;
    const float inv = 1.f / lt;
    TO *op = out + base + (size_t)t * tok;
    // gate values of this lane's outputs (1.0 without a gate), all loads issued first
    uint2 gv[NDT][4];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) gv[dt][g4] = make_uint2(0x3F803F80u, 0x3F803F80u);
    if (gate) {
        const uint16_t *gp = gate + base + (size_t)t * tok;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                gv[dt][g4] = *reinterpret_cast<const uint2 *>(gp + 32 * dt + 8 * g4 + 4 * hh);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            // rows 8 g4 + 4 hh + 0..3 of value tile dt
            const int c = 32 * dt + 8 * g4 + 4 * hh;
            const uint2 g = gv[dt][g4];
            store4<TO>(op + c, oacc[dt][4 * g4 + 0] * inv * __uint_as_float(g.x << 16),
                       oacc[dt][4 * g4 + 1] * inv * __uint_as_float(g.x & 0xFFFF0000u),
                       oacc[dt][4 * g4 + 2] * inv * __uint_as_float(g.y << 16),
                       oacc[dt][4 * g4 + 3] * inv * __uint_as_float(g.y & 0xFFFF0000u));
        }
}

template <int D>
hipError_t launch_swa_d(const SwaArgs &a, hipStream_t s) {
    const int nqt = (a.L + SWA_QT - 1) / SWA_QT;
    const unsigned grid = (unsigned)((size_t)a.B * a.H * nqt);
    const float sl2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
    const uint16_t *q = static_cast<const uint16_t *>(a.q);
    const uint16_t *k = static_cast<const uint16_t *>(a.k);
    const uint16_t *v = static_cast<const uint16_t *>(a.v);
    if (a.out_bf16)
        hipLaunchKernelGGL((swa_fwd_kernel<D, uint16_t>), dim3(grid), dim3(SWA_NTH), 0, s, q, k, v,
                           static_cast<uint16_t *>(a.out), a.gate, a.L, a.H, a.window, nqt, sl2);
    else
        hipLaunchKernelGGL((swa_fwd_kernel<D, float>), dim3(grid), dim3(SWA_NTH), 0, s, q, k, v,
                           static_cast<float *>(a.out), a.gate, a.L, a.H, a.window, nqt, sl2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_swa(const SwaArgs &a, hipStream_t s) {
    if (a.B == 0 || a.L == 0) return hipSuccess;
    return a.d == 64 ? launch_swa_d<64>(a, s) : launch_swa_d<128>(a, s);
}

}  // namespace lt2
