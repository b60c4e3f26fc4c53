// copy.hip -- HBM bandwidth probes (streaming copy, read-only, write-only) and
// state initialisation.
#include "common.h"
#include "internal.h"

namespace lt2 {

// Grid-stride streaming kernels over n 16-byte elements.  Every lane keeps
// UNROLL loads in flight before it consumes them.  MODE 0: copy src -> dst;
// MODE 1: read src only (each lane folds what it read into one value, written
// to dst[global lane] only if the fold equals a value no input produces, so the
// loads cannot be removed and nothing is written in practice); MODE 2: write a
// constant to dst only; MODE 3: copy src -> dst by contiguous tiles of 256 x
// UNROLL elements per workgroup (the access pattern of the decode step's state).
template <int MODE, int UNROLL>
__global__ __launch_bounds__(256) void probe_kernel(f32x4 *__restrict__ dst, const f32x4 *__restrict__ src,
                                                    size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t lane = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if constexpr (MODE == 3) {
        // tiles of 256 * UNROLL consecutive elements, one workgroup each (tiles
        // dealt grid-stride over the workgroups); all loads of a tile are issued
        // before its stores
        const size_t tile = (size_t)blockDim.x * UNROLL;
        for (size_t base = (size_t)blockIdx.x * tile; base < n; base += (size_t)gridDim.x * tile) {
            f32x4 r[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const size_t j = base + (size_t)u * blockDim.x + threadIdx.x;
                if (j < n) r[u] = __builtin_nontemporal_load(src + j);
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const size_t j = base + (size_t)u * blockDim.x + threadIdx.x;
                if (j < n) __builtin_nontemporal_store(r[u], dst + j);
            }
        }
        return;
    }
    size_t i = lane;
    uint32_t fold = 0;
    for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
        f32x4 r[UNROLL];
        if constexpr (MODE != 2) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) r[u] = __builtin_nontemporal_load(src + i + u * stride);
        }
        if constexpr (MODE == 0) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) __builtin_nontemporal_store(r[u], dst + i + u * stride);
        } else if constexpr (MODE == 1) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                fold ^= __float_as_uint(r[u][0]) ^ __float_as_uint(r[u][1]) ^ __float_as_uint(r[u][2]) ^
                        __float_as_uint(r[u][3]);
        } else {
            const f32x4 c = {1.f, 2.f, 3.f, 4.f};
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) __builtin_nontemporal_store(c, dst + i + u * stride);
        }
    }
    for (; i < n; i += stride) {
        if constexpr (MODE == 0) dst[i] = src[i];
        else if constexpr (MODE == 1) fold ^= __float_as_uint(src[i][0]);
        else dst[i] = f32x4{1.f, 2.f, 3.f, 4.f};
    }
    if constexpr (MODE == 1) {
        // 0x7fbadbad is a NaN bit pattern; the probe's callers never read dst in
        // this mode, and lane < n keeps the write inside the buffer
        if (fold == 0x7fbadbadu && lane < n) dst[lane] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

template <int MODE>
static hipError_t probe_u(void *dst, const void *src, size_t n, unsigned blocks, int unroll, hipStream_t s) {
    switch (unroll) {
        case 1: hipLaunchKernelGGL((probe_kernel<MODE, 1>), dim3(blocks), dim3(256), 0, s, (f32x4 *)dst, (const f32x4 *)src, n); break;
        case 2: hipLaunchKernelGGL((probe_kernel<MODE, 2>), dim3(blocks), dim3(256), 0, s, (f32x4 *)dst, (const f32x4 *)src, n); break;
        case 8: hipLaunchKernelGGL((probe_kernel<MODE, 8>), dim3(blocks), dim3(256), 0, s, (f32x4 *)dst, (const f32x4 *)src, n); break;
        case 16: hipLaunchKernelGGL((probe_kernel<MODE, 16>), dim3(blocks), dim3(256), 0, s, (f32x4 *)dst, (const f32x4 *)src, n); break;
        default: hipLaunchKernelGGL((probe_kernel<MODE, 4>), dim3(blocks), dim3(256), 0, s, (f32x4 *)dst, (const f32x4 *)src, n); break;
    }
    return hipGetLastError();
}

hipError_t launch_probe(void *dst, const void *src, size_t bytes, int mode, unsigned blocks, int unroll,
                        hipStream_t s) {
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    if (blocks == 0) blocks = (unsigned)((n + 255) / 256 < 256u * 16u ? (n + 255) / 256 : 256u * 16u);
    switch (mode) {
        case 1: return probe_u<1>(dst, src, n, blocks, unroll, s);
        case 2: return probe_u<2>(dst, src, n, blocks, unroll, s);
        case 3: return probe_u<3>(dst, src, n, blocks, unroll, s);
        default: return probe_u<0>(dst, src, n, blocks, unroll, s);
    }
}

hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s) {
    return launch_probe(dst, src, bytes, 0, 0, 4, s);
}

// dst = src (src != NULL) or dst = 0, n floats.
__global__ __launch_bounds__(256) void state_init_kernel(float *__restrict__ dst, const float *__restrict__ src,
                                                         size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_state_init(float *dst, const float *src, size_t n, hipStream_t s) {
    if (n == 0 || dst == src) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(state_init_kernel, dim3(blocks), dim3(256), 0, s, dst, src, n);
    return hipGetLastError();
}

}  // namespace lt2
