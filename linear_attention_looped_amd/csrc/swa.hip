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
// double-buffered: the next tile is fetched into registers (coalesced 16-byte
// loads) while the current one is used, and written to the other buffer at the
// end of the tile, so one barrier per tile suffices.
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
// fully masked tile contributes exp2(-inf) = 0 without producing NaN.  Masking
// is applied only on tiles that cross the causal diagonal or the window's start;
// tiles wholly outside a wave's range are skipped by that wave.
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

template <int D, typename TO>
__global__ __launch_bounds__(SWA_NTH) __attribute__((amdgpu_waves_per_eu(2, 2)))
void swa_fwd_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                    TO *__restrict__ out, const uint16_t *__restrict__ gate, int L, int H, int window, int nqt,
                    float sl2) {
    constexpr int KT = SWA_KT;
    constexpr int KP = D + 8;          // K row pitch: 16-byte reads of 16 consecutive rows hit distinct banks
    constexpr int VP = D + 32;         // V row pitch: rows 16 banks apart for the transpose reads
    constexpr int NKS = D / 16;        // k-steps of the score product
    constexpr int NDT = D / 32;        // 32-wide value tiles
    constexpr int PPT = KT * D / 8 / SWA_NTH;   // 16-byte pieces per thread per K (or V) tile
    static_assert(PPT * SWA_NTH * 8 == KT * D, "tile pieces");
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][KT * VP];

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

    // Q^T fragments: B operand of S^T = K Q^T, query l32, channels 16 ks + 8 hh .. + 7
    bf16x8 qf[NKS];
    {
        const uint16_t *qp = q + base + (size_t)tq * tok + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
    }

    // staging roles: piece p = tid + 256 i is row p / (D/8), 8 channels at 8 (p % (D/8))
    int srow[PPT], scol[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = tid + SWA_NTH * i;
        srow[i] = p / (D / 8);
        scol[i] = 8 * (p % (D / 8));
    }
    u32x4 rk[PPT], rv[PPT];
    auto fetch = [&](int kt) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const size_t row = (size_t)min(kt * KT + srow[i], L - 1);
            rk[i] = *reinterpret_cast<const u32x4 *>(k + base + row * tok + scol[i]);
            rv[i] = *reinterpret_cast<const u32x4 *>(v + base + row * tok + scol[i]);
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            *reinterpret_cast<u32x4 *>(&Ks[buf][srow[i] * KP + scol[i]]) = rk[i];
            *reinterpret_cast<u32x4 *>(&Vs[buf][srow[i] * VP + scol[i]]) = rv[i];
        }
    };

    fetch(kt0);
    stage(0);
    __syncthreads();

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m = -1e30f, lsum = 0.f;
    // transpose-read roles: within each 16-lane group, lane 4e + c addresses row
    // e of a 4-row block at channel 4c; the group's second bit picks the 16-channel half
    const int tr_e = (lane & 15) >> 2;
    const int tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    for (int kt = kt0; kt <= kt1; ++kt) {
        const int buf = (kt - kt0) & 1;
        if (kt < kt1) fetch(kt + 1);
        const int ka = kt * KT;
        const bool active = wave_live && ka <= qlast && ka + KT - 1 >= qa - window + 1;
        if (active) {
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
                const uint16_t *kr = &Ks[buf][(32 * kb + l32) * KP + 8 * hh];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kr + 16 * ks);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
                }
            }
            // every key of the tile inside every live query's window?
            const bool full = ka + KT - 1 <= qa && ka >= qlast - window + 1;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = s[kb][r];
                    if (!full) {
                        const int j = ka + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                        if (j > tq || j <= tq - window) x = -INFINITY;
                    }
                    s[kb][r] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m, mx * sl2);
            const float f = __builtin_amdgcn_exp2f(m - mnew);
            m = mnew;
            lsum *= f;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= f;
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
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    // keys 32 kb + 16 hf + 4 hh + 0..3 (slots 0-3) and + 8 (slots 4-7)
                    const int r0 = 32 * kb + 16 * hf + 4 * hh + tr_e;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        const short4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_short4 *)(&Vs[buf][r0 * VP + 32 * dt + tr_c]));
                        const short4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_short4 *)(&Vs[buf][(r0 + 8) * VP + 32 * dt + tr_c]));
                        const bf16x8 a = __builtin_bit_cast(
                            bf16x8, (__attribute__((ext_vector_type(8))) short){lo4[0], lo4[1], lo4[2], lo4[3],
                                                                                hi4[0], hi4[1], hi4[2], hi4[3]});
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][hf], oacc[dt], 0, 0, 0);
                    }
                }
        }
        if (kt < kt1) {
            wait_vmem_all();
            stage(buf ^ 1);
        }
        __syncthreads();
    }

    if (!wave_live) return;
    const float lt = lsum + __shfl_xor(lsum, 32);
    const int t = qa + l32;
    if (t >= L) return;
    const float inv = 1.f / lt;
    TO *op = out + base + (size_t)t * tok;
    const uint16_t *gp = gate ? gate + base + (size_t)t * tok : nullptr;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            // rows 8 g4 + 4 hh + 0..3 of value tile dt
            const int c = 32 * dt + 8 * g4 + 4 * hh;
            float o0 = oacc[dt][4 * g4 + 0] * inv, o1 = oacc[dt][4 * g4 + 1] * inv;
            float o2 = oacc[dt][4 * g4 + 2] * inv, o3 = oacc[dt][4 * g4 + 3] * inv;
            if (gp) {
                const uint2 g = *reinterpret_cast<const uint2 *>(gp + c);
                o0 *= __uint_as_float(g.x << 16);
                o1 *= __uint_as_float(g.x & 0xFFFF0000u);
                o2 *= __uint_as_float(g.y << 16);
                o3 *= __uint_as_float(g.y & 0xFFFF0000u);
            }
            store4<TO>(op + c, o0, o1, o2, o3);
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
