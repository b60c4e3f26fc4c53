// copy.hip -- streaming copy (HBM bandwidth probe) and state initialisation.
#include "common.h"
#include "internal.h"

namespace lt2 {

// Grid-stride 16-byte copy; every lane moves UNROLL float4 per iteration so
// that several loads are in flight before the stores.
__global__ __launch_bounds__(256) void copy_kernel(f32x4 *__restrict__ dst, const f32x4 *__restrict__ src,
                                                   size_t n) {
    constexpr int UNROLL = 4;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
        f32x4 r[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) r[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) __builtin_nontemporal_store(r[u], dst + i + u * stride);
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 256u * 16u ? (n + 255) / 256 : 256u * 16u);
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, s, (f32x4 *)dst, (const f32x4 *)src, n);
    return hipGetLastError();
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
