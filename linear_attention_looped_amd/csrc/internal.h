// internal.h -- launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lt2 {

// Compute units of the current device (cached per device).
inline int device_cus() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
    }
    return cus[dev];
}

struct GdnArgs {
    int B, L, H, dk, dv, chunk;
    int qkv_bf16, out_bf16, channel;
    const void *q, *k, *v;
    const float *alpha, *beta;
    const float *state_in;
    void *out;
    float *state_out;
    void *ws;
    // Looped block only: bf16 output gate (same layout as out), multiplied into
    // the output by the scalar-gate bf16 scan and the decode step; nullptr = none.
    const uint16_t *gate = nullptr;
};

// Each launcher returns hipSuccess or the launch error; shapes are already
// validated by the caller.
// Prefill phases: the chunk-parallel prepare phase writes the per-chunk
// factors into the workspace, the scan phase carries the state across chunks.
enum { PHASE_PREPARE = 1, PHASE_SCAN = 2, PHASE_ALL = 3 };

hipError_t launch_decode(const GdnArgs &a, hipStream_t s);
size_t prefill_head_ws_bytes(int B, int L, int H, int C);
hipError_t launch_prefill_head(const GdnArgs &a, int phase, hipStream_t s);
size_t prefill_channel_ws_bytes(int B, int L, int H, int dk, int C, bool bf16);
hipError_t launch_prefill_channel(const GdnArgs &a, int phase, hipStream_t s);
hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s);
hipError_t launch_probe(void *dst, const void *src, size_t bytes, int mode, unsigned blocks, int unroll,
                        hipStream_t s);

// Causal sliding-window softmax attention: q, k, v bf16 [B, L, H, d], out bf16
// or fp32 [B, L, H, d], keys t-window+1 .. t for query t, scale 1/sqrt(d);
// gate (bf16, out's layout, or nullptr) multiplies the output where it is stored.
struct SwaArgs {
    int B, L, H, d, window, out_bf16;
    const void *q, *k, *v;
    void *out;
    const uint16_t *gate = nullptr;
};
hipError_t launch_swa(const SwaArgs &a, hipStream_t s);

// One decode token of the window mixer against per-(b, h) rings of w keys/values.
struct SwaDecodeArgs {
    int B, H, d, window, out_bf16;
    const void *q, *k, *v;
    void *k_cache, *v_cache;
    const int32_t *pos;
    void *out;
    const uint16_t *gate = nullptr;   // [B, H, d] bf16 output gate, or null
};
hipError_t launch_swa_decode(const SwaDecodeArgs &a, hipStream_t s);

// Backward pass of the gated-delta prefill, scalar gate; gradients fp32.
struct GdnBwdArgs {
    int B, L, H, d, qkv_bf16, dout_bf16;
    const void *q, *k, *v;
    const float *alpha, *beta;
    const float *state_in;      // [B, H, d, d] or nullptr (zero)
    const void *dout;           // [B, L, H, d], bf16 or fp32
    const float *dstate_out;    // [B, H, d, d] or nullptr (zero)
    float *dq, *dk, *dv;        // [B, L, H, d]
    float *dlog_alpha, *dbeta;  // [B, L, H]
    float *dstate_in;           // [B, H, d, d] or nullptr
    void *ws;
};
size_t gdn_bwd_ws_bytes(int B, int L, int H, int d);
hipError_t launch_gdn_bwd(const GdnBwdArgs &a, hipStream_t s);
// Per-channel gate: dlog_alpha is [B, L, H, d].
size_t kda_bwd_ws_bytes(int B, int L, int H, int d);
hipError_t launch_kda_bwd(const GdnBwdArgs &a, hipStream_t s);

// Looped LT2-linear block.
struct LoopArgs {
    int B, L, D, H, d, T, chunk, gated;
    const float *h_in;
    float *h_out;
    const uint16_t *W_in, *W_o;
    void *ws;
};
// Byte offsets of the looped block's buffers inside its workspace.
struct LoopLayout {
    size_t xb, q, k, v, g, beta, alpha, o, prefill, total;
};
LoopLayout loop_layout(int B, int L, int D, int H, int d, int chunk, bool gated);
hipError_t launch_looped(const LoopArgs &a, hipStream_t s);

// Looped hybrid block: a shared stack of layers (gated-delta or window
// attention), applied in order, T times.
constexpr int HYBRID_MAX_LAYERS = 8;
struct HybridArgs {
    int B, L, D, H, d, T, chunk, gated, window, n_layers;
    int kinds[HYBRID_MAX_LAYERS];                 // 0 gated delta, 1 window attention
    const float *h_in;
    float *h_out;
    const uint16_t *W_in[HYBRID_MAX_LAYERS], *W_o[HYBRID_MAX_LAYERS];
    void *ws;
};
hipError_t launch_hybrid(const HybridArgs &a, hipStream_t s);

// Looped decode: one token per sequence, T loop states carried in place.
struct LoopDecodeArgs {
    int B, D, H, d, T, gated;
    float *h;                // [B, D] fp32, in place
    const uint16_t *W_in, *W_o;
    float *states;           // [T, B, H, d, d] fp32, in place
    void *ws;
};
LoopLayout loop_decode_layout(int B, int D, int H, int d, bool gated);
hipError_t launch_looped_decode(const LoopDecodeArgs &a, hipStream_t s);

// Looped hybrid decode: one token per sequence through T loops of the layer
// stack; gated-delta layer states and window-layer rings per (loop, layer).
struct HybridDecodeArgs {
    int B, D, H, d, T, gated, window, n_layers;
    int kinds[HYBRID_MAX_LAYERS];
    float *h;                          // [B, D] fp32, in place
    const uint16_t *W_in[HYBRID_MAX_LAYERS], *W_o[HYBRID_MAX_LAYERS];
    float *states;                     // [T, n_gdn, B, H, d, d] fp32
    uint16_t *k_rings, *v_rings;       // [T, n_swa, B, H, window, d] bf16
    const int32_t *pos;                // [B]
    void *ws;
};
hipError_t launch_hybrid_decode(const HybridDecodeArgs &a, hipStream_t s);
hipError_t launch_state_init(float *dst, const float *src, size_t n, hipStream_t s);

}  // namespace lt2
