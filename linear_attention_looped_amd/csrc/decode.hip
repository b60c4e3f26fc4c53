// decode.hip -- one decode token of the gated delta rule, state updated in place.
//
// LT2 explainer (paithon.it), "Sostituire il motore", state-update equation:
//   S' = Diag(alpha)(S - beta k (k^T S)) + beta k v^T,   o = S'^T q.
// The read-out is taken from the OLD state in the same pass:
//   o = S^T(alpha*q) - beta (q.(alpha*k)) S^T k + beta (q.k) v,
// so the d_k x d_v fp32 state is read once and written once.
//
// One workgroup (256 lanes) per (b, h) unit, each streaming its own contiguous
// state block.  Lane (rg, cg) owns four adjacent
// columns 4cg..4cg+3 of rows rg, rg+RG, rg+2RG, ...: for every row step the
// 256 lanes cover RG consecutive rows, one contiguous block of RG*d_v*4 bytes.
// Column sums of k^T S and (alpha*q)^T S are reduced over the RG row groups in
// LDS; q.k and q.(alpha*k) are reduced by wave 0 meanwhile.
#include "common.h"
#include "internal.h"

namespace lt2 {

template <typename T>
__device__ __forceinline__ float4 load4(const T *p);
template <>
__device__ __forceinline__ float4 load4<float>(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}
template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t *p) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}
template <typename T>
__device__ __forceinline__ void store4(T *p, float4 x);
template <>
__device__ __forceinline__ void store4<float>(float *p, float4 x) {
    *reinterpret_cast<float4 *>(p) = x;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t *p, float4 x) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16(x.x) | ((uint32_t)f32_to_bf16(x.y) << 16);
    u.y = (uint32_t)f32_to_bf16(x.z) | ((uint32_t)f32_to_bf16(x.w) << 16);
    *reinterpret_cast<uint2 *>(p) = u;
}

template <int DK, int DV, bool CHANNEL, typename TI, typename TO>
__global__ __launch_bounds__(256) void gdn_decode_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                         const TI *__restrict__ v,
                                                         const float *__restrict__ alpha,
                                                         const float *__restrict__ beta,
                                                         float *__restrict__ state, TO *__restrict__ out,
                                                         const uint16_t *__restrict__ gate) {
    constexpr int CG = DV / 4;     // float4 column groups per row
    constexpr int RG = 256 / CG;   // row groups
    constexpr int RPT = DK / RG;   // rows per lane
    static_assert(256 % CG == 0 && DK % RG == 0, "decode tiling");

    __shared__ float sq[DK], sk[DK], sa[DK];
    __shared__ float4 red_k[RG][CG], red_q[RG][CG];
    __shared__ float sdot[2];

    const size_t u = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;

    // The state's loads go out first (they do not wait for q, k and alpha).
    // State loads and stores carry the non-temporal hint: each state block is
    // touched once per launch, and with both hints the stream measured 92.5 us
    // per 4096-unit launch against 106.7 us with neither (a non-temporal store
    // alone was slower, 108.1 us).
    float *S = state + u * (size_t)(DK * DV);
    float4 s[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int row = rg + j * RG;
        s[j] = __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + row * DV + 4 * cg)));
    }
    for (int i = tid; i < DK; i += 256) {
        sq[i] = load1<TI>(q + u * DK + i);
        sk[i] = load1<TI>(k + u * DK + i);
        sa[i] = CHANNEL ? alpha[u * DK + i] : alpha[u];
    }
    __syncthreads();

    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int row = rg + j * RG;
        const float kr = sk[row], qr = sq[row] * sa[row];
        pk.x += kr * s[j].x; pk.y += kr * s[j].y; pk.z += kr * s[j].z; pk.w += kr * s[j].w;
        pq.x += qr * s[j].x; pq.y += qr * s[j].y; pq.z += qr * s[j].z; pq.w += qr * s[j].w;
    }
    red_k[rg][cg] = pk;
    red_q[rg][cg] = pq;
    if (tid < 64) {
        float d0 = 0.f, d1 = 0.f;
        for (int i = tid; i < DK; i += 64) {
            const float qk = sq[i] * sk[i];
            d0 += qk;
            d1 += qk * sa[i];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            d0 += __shfl_xor(d0, off);
            d1 += __shfl_xor(d1, off);
        }
        if (tid == 0) { sdot[0] = d0; sdot[1] = d1; }
    }
    __syncthreads();

    float4 kS = red_k[0][cg], qS = red_q[0][cg];
#pragma unroll
    for (int r = 1; r < RG; ++r) {
        const float4 a = red_k[r][cg], b = red_q[r][cg];
        kS.x += a.x; kS.y += a.y; kS.z += a.z; kS.w += a.w;
        qS.x += b.x; qS.y += b.y; qS.z += b.z; qS.w += b.w;
    }
    const float bt = beta[u];
    const float cq = bt * sdot[1];   // beta * q.(alpha*k)
    const float cv = bt * sdot[0];   // beta * q.k
    const float4 vv = load4<TI>(v + u * DV + 4 * cg);
    if (rg == 0) {
        float4 o;
        o.x = qS.x - cq * kS.x + cv * vv.x;
        o.y = qS.y - cq * kS.y + cv * vv.y;
        o.z = qS.z - cq * kS.z + cv * vv.z;
        o.w = qS.w - cq * kS.w + cv * vv.w;
        if (gate) {   // output gate of the looped block: o * sigmoid(z_g), bf16 gate values
            const float4 gv = load4<uint16_t>(gate + u * DV + 4 * cg);
            o.x *= gv.x; o.y *= gv.y; o.z *= gv.z; o.w *= gv.w;
        }
        store4<TO>(out + u * DV + 4 * cg, o);
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int row = rg + j * RG;
        const float a = sa[row], bk = bt * sk[row];
        float4 n;
        n.x = a * (s[j].x - bk * kS.x) + bk * vv.x;
        n.y = a * (s[j].y - bk * kS.y) + bk * vv.y;
        n.z = a * (s[j].z - bk * kS.z) + bk * vv.z;
        n.w = a * (s[j].w - bk * kS.w) + bk * vv.w;
        __builtin_nontemporal_store(__builtin_bit_cast(f32x4, n), reinterpret_cast<f32x4 *>(S + row * DV + 4 * cg));
    }
}

template <int D, bool CH, typename TI, typename TO>
static hipError_t dec(const GdnArgs &a, hipStream_t s) {
    const unsigned units = (unsigned)a.B * (unsigned)a.H;
    hipLaunchKernelGGL((gdn_decode_kernel<D, D, CH, TI, TO>), dim3(units), dim3(256), 0, s,
                       (const TI *)a.q, (const TI *)a.k, (const TI *)a.v, a.alpha, a.beta, a.state_out,
                       (TO *)a.out, a.gate);
    return hipGetLastError();
}

template <int D, bool CH>
static hipError_t dec_t(const GdnArgs &a, hipStream_t s) {
    if (a.qkv_bf16) return a.out_bf16 ? dec<D, CH, uint16_t, uint16_t>(a, s) : dec<D, CH, uint16_t, float>(a, s);
    return a.out_bf16 ? dec<D, CH, float, uint16_t>(a, s) : dec<D, CH, float, float>(a, s);
}

hipError_t launch_decode(const GdnArgs &a, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    if (a.dk == 64) return a.channel ? dec_t<64, true>(a, s) : dec_t<64, false>(a, s);
    return a.channel ? dec_t<128, true>(a, s) : dec_t<128, false>(a, s);
}

}  // namespace lt2
