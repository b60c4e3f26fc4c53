// gemm.h -- launchers of the bf16 GEMM with the looped block's epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lt2 {

enum { EPI_PROJ = 0, EPI_RESID = 1 };

// [q|k|v(|g)|beta|alpha] = X W^T with per-head L2 norm of q, k (norm_qk), the
// output gate g = sigmoid(z_g) (bf16, when g != nullptr) and the gate
// transforms (when beta != nullptr); X [M, K] bf16, W [N, K] bf16 with
// N = 3*H*d + 2*H (4*H*d + 2*H with g), or 3*H*d (4*H*d) without beta/alpha.
hipError_t launch_gemm_proj(const uint16_t *X, const uint16_t *W, int M, int N, int K, uint16_t *q, uint16_t *k,
                            uint16_t *v, uint16_t *g, float *beta, float *alpha, int H, int d, hipStream_t s,
                            bool norm_qk = true);
// h += O W^T (fp32, in place) and xb = bf16(h); O [M, K] bf16, W [N, K] bf16.
hipError_t launch_gemm_resid(const uint16_t *O, const uint16_t *W, int M, int N, int K, float *h, uint16_t *xb,
                             hipStream_t s);
// h_out = h_in (if distinct) and xb = bf16(h_in), n floats (multiple of 4).
hipError_t launch_cast_residual(const float *h_in, float *h_out, uint16_t *xb, size_t n, hipStream_t s);

}  // namespace lt2
