// common.h -- device helpers shared by the gfx950 kernels of liblt2.
//
// Matrix-core (MFMA) fragments.  Every contraction is cut into 16x16 output
// tiles and K-blocks of 32.  For one K-block each lane of a 64-wide wave holds
// eight consecutive K values of one A row and of one B column:
//     A[i][k]: lane = i + 16*(k/8), slot k%8     (i < 16, k < 32)
//     B[k][j]: lane = j + 16*(k/8), slot k%8
// and the accumulator holds D[4*(lane/16) + r][lane%16] in register r.
// That is the operand layout of v_mfma_f32_16x16x32_bf16.  The fp32 path
// issues eight v_mfma_f32_16x16x4_f32 over the same fragments (slot s of every
// lane in instruction s), which sums the same 32 products in another order.
//
// bf16 operands that are not exactly representable (fp32 intermediates such
// as the state) are split into hi = bf16(x) and lo = bf16(x - hi); a product
// then takes hi*hi + lo*hi + hi*lo, which keeps about 16 significant bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lt2 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

enum Prec { PREC_F32 = 0, PREC_BF16 = 1 };

struct Frag {
    float x[8];
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void split_bf16(const Frag &a, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        __bf16 h = (__bf16)a.x[e];
        hi[e] = h;
        lo[e] = (__bf16)(a.x[e] - (float)h);
    }
}

__device__ __forceinline__ void to_bf16(const Frag &a, bf16x8 &hi) {
#pragma unroll
    for (int e = 0; e < 8; ++e) hi[e] = (__bf16)a.x[e];
}

// acc += A-block * B-block for one K-block of 32.
// A_EXACT / B_EXACT: the operand holds bf16-representable values (inputs).
template <int PREC, bool A_EXACT, bool B_EXACT>
__device__ __forceinline__ void mma(f32x4 &acc, const Frag &a, const Frag &b) {
    if constexpr (PREC == PREC_F32) {
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x[s], b.x[s], acc, 0, 0, 0);
    } else {
        bf16x8 ah, al, bh, bl;
        if constexpr (A_EXACT) to_bf16(a, ah); else split_bf16(a, ah, al);
        if constexpr (B_EXACT) to_bf16(b, bh); else split_bf16(b, bh, bl);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        if constexpr (!A_EXACT) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
        if constexpr (!B_EXACT) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    }
}

// Pre-converted MFMA operands, so one fragment can feed several products
// without repeating the conversion.  fp32 path: the eight floats; bf16 path:
// hi (and lo for operands that are not bf16-exact).
template <int PREC, bool EXACT>
struct Op {
    bf16x8 hi, lo;
};
template <bool EXACT>
struct Op<PREC_F32, EXACT> {
    Frag f;
};

template <int PREC, bool EXACT>
__device__ __forceinline__ Op<PREC, EXACT> make_op(const Frag &a) {
    Op<PREC, EXACT> o;
    if constexpr (PREC == PREC_F32) {
        o.f = a;
    } else if constexpr (EXACT) {
        to_bf16(a, o.hi);
    } else {
        split_bf16(a, o.hi, o.lo);
    }
    return o;
}

template <int PREC, bool AE, bool BE>
__device__ __forceinline__ void mma_op(f32x4 &acc, const Op<PREC, AE> &a, const Op<PREC, BE> &b) {
    if constexpr (PREC == PREC_F32) {
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f.x[s], b.f.x[s], acc, 0, 0, 0);
    } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
        if constexpr (!AE) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
        if constexpr (!BE) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    }
}

// Raw eight-element input rows (kept in their storage type while in flight).
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
    uint4 u;
};
template <>
struct Raw8<float> {
    float4 a, b;
};

template <typename T>
__device__ __forceinline__ void load_raw8(Raw8<T> &r, const T *p);
template <>
__device__ __forceinline__ void load_raw8<uint16_t>(Raw8<uint16_t> &r, const uint16_t *p) {
    r.u = *reinterpret_cast<const uint4 *>(p);
}
template <>
__device__ __forceinline__ void load_raw8<float>(Raw8<float> &r, const float *p) {
    r.a = *reinterpret_cast<const float4 *>(p);
    r.b = *reinterpret_cast<const float4 *>(p + 4);
}

template <typename T>
__device__ __forceinline__ void zero_raw8(Raw8<T> &r);
template <>
__device__ __forceinline__ void zero_raw8<uint16_t>(Raw8<uint16_t> &r) {
    r.u = make_uint4(0u, 0u, 0u, 0u);
}
template <>
__device__ __forceinline__ void zero_raw8<float>(Raw8<float> &r) {
    r.a = make_float4(0.f, 0.f, 0.f, 0.f);
    r.b = r.a;
}

__device__ __forceinline__ void raw_to_frag(Frag &f, const Raw8<uint16_t> &r) {
    const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.x[2 * i] = __uint_as_float(w[i] << 16);
        f.x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void raw_to_frag(Frag &f, const Raw8<float> &r) {
    f.x[0] = r.a.x; f.x[1] = r.a.y; f.x[2] = r.a.z; f.x[3] = r.a.w;
    f.x[4] = r.b.x; f.x[5] = r.b.y; f.x[6] = r.b.z; f.x[7] = r.b.w;
}

// Wait until every outstanding vector-memory load of this wave has landed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt untouched).  Placed where prefetched
// data is known to have had time to arrive, it also gives the compiler's
// wait-count tracking a clean state across a loop back-edge, so later uses of
// the prefetched registers do not wait on loads issued after them.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations still
// outstanding (they retire in issue order); expcnt and lgkmcnt untouched.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
}

// The hardware hands out the workgroups of a launch to the 8 XCDs (each with
// its own L2) round-robin by workgroup id.  This maps a 1-D id to a logical
// index so that the ids one XCD receives get consecutive logical indices, i.e.
// neighbouring logical work (which shares inputs) lands on the same L2.
__device__ __forceinline__ int xcd_logical(int bid, int n) {
    if (n % 8 != 0) return bid;
    return (bid % 8) * (n / 8) + bid / 8;
}

// Fragment loads: eight consecutive floats from a row of an fp32 buffer.
__device__ __forceinline__ void load_frag_f32(Frag &f, const float *p) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    f.x[0] = a.x; f.x[1] = a.y; f.x[2] = a.z; f.x[3] = a.w;
    f.x[4] = b.x; f.x[5] = b.y; f.x[6] = b.z; f.x[7] = b.w;
}

// Eight floats with a stride (column of a row-major LDS buffer).
__device__ __forceinline__ void load_frag_strided(Frag &f, const float *p, int stride) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.x[e] = p[e * stride];
}

__device__ __forceinline__ void zero_frag(Frag &f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.x[e] = 0.f;
}

// Eight consecutive elements of a global input row, widened to fp32.
template <typename T>
__device__ __forceinline__ void load_row8(Frag &f, const T *p);

template <>
__device__ __forceinline__ void load_row8<float>(Frag &f, const float *p) {
    load_frag_f32(f, p);
}

template <>
__device__ __forceinline__ void load_row8<uint16_t>(Frag &f, const uint16_t *p) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.x[2 * i] = __uint_as_float(w[i] << 16);
        f.x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <typename T>
__device__ __forceinline__ float load1(const T *p);
template <>
__device__ __forceinline__ float load1<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }

template <typename T>
__device__ __forceinline__ void store1(T *p, float x);
template <>
__device__ __forceinline__ void store1<float>(float *p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store1<uint16_t>(uint16_t *p, float x) { *p = f32_to_bf16(x); }

// log2(alpha) with alpha = 0 mapped to a finite -116 (a factor below 2e-35).
// Gates are carried in base 2 so that every decay factor is one v_exp_f32.
__device__ __forceinline__ float log2_gate(float a) {
    return fmaxf(__builtin_amdgcn_logf(fmaxf(a, 1e-38f)), -116.f);
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// x computed where it stands, for every lane: the compiler may not sink the work
// behind it into the arm of a later select (it turns such a select of a value
// fed by a one-use LDS load into a branch per element, serialising load, wait
// and exp).  An empty asm with x as a register operand; no instruction.
__device__ __forceinline__ float materialize(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// fp32 -> bf16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
// Two fp32 values -> packed bf16 hi = bf16(x) and lo = bf16(x - hi), both
// rounded to nearest even; one two-value conversion instruction per pair.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    typedef __attribute__((ext_vector_type(2))) float f2_t;
    typedef __attribute__((ext_vector_type(2))) __bf16 b2_t;
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, b2_t));
    const float ha = __uint_as_float(h << 16), hb = __uint_as_float(h & 0xFFFF0000u);
    hi = h;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a - ha, b - hb}, b2_t));
}
// Four fp32 values -> bf16 hi and lo = bf16(x - hi), each packed in a uint2.
__device__ __forceinline__ void split4(const float x[4], uint2 &hi, uint2 &lo) {
    split2(x[0], x[1], hi.x, lo.x);
    split2(x[2], x[3], hi.y, lo.y);
}
// Eight fp32 values -> bf16 hi and lo, each packed in a uint4.
__device__ __forceinline__ void split8(const float x[8], uint4 &hi, uint4 &lo) {
    uint2 h0, l0, h1, l1;
    split4(x, h0, l0);
    split4(x + 4, h1, l1);
    hi = make_uint4(h0.x, h0.y, h1.x, h1.y);
    lo = make_uint4(l0.x, l0.y, l1.x, l1.y);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

}  // namespace lt2
