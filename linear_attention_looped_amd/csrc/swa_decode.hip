// swa_decode.hip -- one decode token of the causal sliding-window mixer (LT2
// explainer, paithon.it, section "Sostituire il motore": each token attends to
// a window of the w most recent positions, itself included).  The window is a
// ring of the last w keys and values per (b, h): the new token's key and value
// go to slot pos mod w, and its query attends to every filled slot (the tokens
// max(0, pos-w+1) .. pos; the softmax does not depend on their order):
//
//   o = sum_j softmax_j(q . k_j / sqrt(d)) v_j
//
// One workgroup of 256 lanes per (b, h).  Groups of G = d/8 lanes take one key
// at a time (16 bytes of bf16 per lane, so a group reads a whole key and value
// row with one coalesced access each), keys j = g, g + NG, ... for group g;
// each group keeps an online softmax (running maximum, sum and its lanes' eight
// output channels) in base 2, the score scale log2(e)/sqrt(d) folded into q.
// The groups' partial results meet in LDS at the end.  The ring is streamed
// once (2 w d bytes of bf16 per (b, h) and token): the kernel is HBM-bound and
// reads nearly only, so its ceiling is the read stream's.
//
// The new key and value are written to their slot and also kept in LDS; a
// group reading that slot takes the LDS copy, so no lane depends on seeing the
// other lanes' global write in this launch.
#include "common.h"
#include "internal.h"

namespace lt2 {

namespace {

__device__ __forceinline__ void unpack8(const uint4 &u, float (&x)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <typename TO>
__device__ __forceinline__ TO to_out(float x);
template <>
__device__ __forceinline__ float to_out<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t to_out<uint16_t>(float x) { return f32_to_bf16(x); }

template <int D, typename TO>
__global__ __launch_bounds__(256) void swa_decode_kernel(const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v, uint16_t *__restrict__ kc,
                                                         uint16_t *__restrict__ vc, const int32_t *__restrict__ pos,
                                                         TO *__restrict__ out, int H, int W, float qscale,
                                                         const uint16_t *__restrict__ gate) {
    constexpr int G = D / 8;       // lanes per key
    constexpr int NG = 256 / G;    // key groups
    static_assert(64 % G == 0, "a key group lies within one wave");
    __shared__ float qs[D];
    __shared__ uint4 knew[G], vnew[G];
    __shared__ float gmax[NG], gsum[NG];
    __shared__ float gacc[NG][D + 4];

    const size_t unit = blockIdx.x;
    const int b = (int)(unit / (size_t)H);
    const int tid = threadIdx.x, grp = tid / G, gl = tid % G;
    const int p = max(pos[b], 0);
    const int slot = p % W;
    const int n = min(p, W - 1) + 1;                 // filled slots 0 .. n-1
    const size_t ring = unit * (size_t)W * D;        // element offset of this unit's ring

    if (tid < D) qs[tid] = bf16_to_f32(q[unit * D + tid]) * qscale;
    if (tid < G) {
        const uint4 kn = reinterpret_cast<const uint4 *>(k + unit * D)[tid];
        const uint4 vn = reinterpret_cast<const uint4 *>(v + unit * D)[tid];
        knew[tid] = kn;
        vnew[tid] = vn;
        reinterpret_cast<uint4 *>(kc + ring + (size_t)slot * D)[tid] = kn;
        reinterpret_cast<uint4 *>(vc + ring + (size_t)slot * D)[tid] = vn;
    }
    __syncthreads();

    float qr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[e] = qs[8 * gl + e];
    const uint4 kn = knew[gl], vn = vnew[gl];
    float m = -1e30f, l = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const uint4 *kr = reinterpret_cast<const uint4 *>(kc + ring) + gl;
    const uint4 *vr = reinterpret_cast<const uint4 *>(vc + ring) + gl;
    // each group's next key and value are loaded one step ahead, with the
    // non-temporal hint (each ring row is read once per launch): 189.8 -> 170.1
    // us on 256 x 16 rings of 512 (loading a second key ahead: 172.8 us)
    uint4 kp = kn, vp = vn;
    if (grp < n) {
        kp = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kr + (size_t)grp * G)));
        vp = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vr + (size_t)grp * G)));
    }
    for (int j = grp; j < n; j += NG) {
        uint4 ku = kp, vu = vp;
        if (j + NG < n) {
            kp = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kr + (size_t)(j + NG) * G)));
            vp = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vr + (size_t)(j + NG) * G)));
        }
        if (j == slot) {   // uniform over the group
            ku = kn;
            vu = vn;
        }
        float kx[8], vx[8];
        unpack8(ku, kx);
        unpack8(vu, vx);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += qr[e] * kx[e];
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
        const float mn = fmaxf(m, s);
        const float c = exp2_fast(m - mn), w = exp2_fast(s - mn);
        l = l * c + w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] * c + w * vx[e];
        m = mn;
    }
    if (gl == 0) {
        gmax[grp] = m;
        gsum[grp] = l;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) gacc[grp][8 * gl + e] = acc[e];
    __syncthreads();

    if (tid < D) {
        float M = gmax[0];
#pragma unroll
        for (int g = 1; g < NG; ++g) M = fmaxf(M, gmax[g]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float f = exp2_fast(gmax[g] - M);   // zero for groups that saw no key
            num += f * gacc[g][tid];
            den += f * gsum[g];
        }
        float o = num / den;
        if (gate) o *= bf16_to_f32(gate[unit * D + tid]);   // output gate of the looped hybrid block
        out[unit * D + tid] = to_out<TO>(o);
    }
}

template <int D>
hipError_t launch_d(const SwaDecodeArgs &a, hipStream_t s) {
    const unsigned grid = (unsigned)((size_t)a.B * a.H);
    const float qscale = 1.4426950408889634f / sqrtf((float)D);
    if (a.out_bf16)
        hipLaunchKernelGGL((swa_decode_kernel<D, uint16_t>), dim3(grid), dim3(256), 0, s, (const uint16_t *)a.q,
                           (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.k_cache,
                           (uint16_t *)a.v_cache, a.pos, (uint16_t *)a.out, a.H, a.window, qscale,
                           a.gate);
    else
        hipLaunchKernelGGL((swa_decode_kernel<D, float>), dim3(grid), dim3(256), 0, s, (const uint16_t *)a.q,
                           (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.k_cache,
                           (uint16_t *)a.v_cache, a.pos, (float *)a.out, a.H, a.window, qscale,
                           a.gate);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_swa_decode(const SwaDecodeArgs &a, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    return a.d == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace lt2
