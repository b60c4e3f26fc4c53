// api.hip -- extern "C" entry points of liblt2.so (declared in include/lt2.h).
//
// Every entry point validates its whole argument list on the host before it
// enqueues anything, so an error leaves all outputs untouched.
#include "lt2.h"

#include <mutex>

#include "internal.h"

using namespace lt2;

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Every launch of the gated-delta kernels has one workgroup per (unit, chunk)
// (prepare, backward gradients: at most 512 threads), per (unit, column block
// of >= 16 columns) (scans, the per-channel backward: at most 1024 threads) or
// per unit (decode); the runtime rejects a launch of 2^32 threads or more.
// Checked here in 64 bits, before anything is enqueued, for `units` (b, h)
// units of L tokens in chunks of `chunk` (the backward pass always uses 64, at
// least the smallest chunk, 16).
bool launch_fits(int64_t units, int64_t L, int64_t chunk, bool decode = false) {
    if (decode) return units <= 0xffffffffLL / 256;   // 256 threads per unit
    const int64_t chunks = units * ((L + chunk - 1) / chunk);
    const int64_t col_blocks = units * (128 / 16);
    return chunks <= 0xffffffffLL / 512 && col_blocks <= 0xffffffffLL / 1024;
}

lt2_status check_desc(const lt2_gdn_desc *d, bool decode) {
    if (!d) return LT2_ERR_NULL;
    if (d->B < 0 || d->L < 0 || d->H <= 0 || d->d_k <= 0 || d->d_v <= 0) return LT2_ERR_SHAPE;
    if (decode && d->L != 1) return LT2_ERR_SHAPE;
    if ((d->qkv_dtype != LT2_F32 && d->qkv_dtype != LT2_BF16) ||
        (d->out_dtype != LT2_F32 && d->out_dtype != LT2_BF16))
        return LT2_ERR_DTYPE;
    if (d->gate != LT2_GATE_HEAD && d->gate != LT2_GATE_CHANNEL) return LT2_ERR_UNSUPPORTED;
    if (d->d_k != d->d_v || (d->d_k != 64 && d->d_k != 128)) return LT2_ERR_UNSUPPORTED;
    if (!decode && d->chunk != 16 && d->chunk != 32 && d->chunk != 64) return LT2_ERR_UNSUPPORTED;
    // index arithmetic inside the kernels is 64-bit for element offsets; the
    // grid dimensions must fit their 32-bit and 65535 limits
    if ((int64_t)d->B * d->H > 0x7fffffffLL) return LT2_ERR_SHAPE;
    if (!decode && (d->H > 65535 || d->B > 65535)) return LT2_ERR_SHAPE;
    if (!launch_fits((int64_t)d->B * d->H, d->L, decode ? 1 : d->chunk, decode)) return LT2_ERR_SHAPE;
    return LT2_OK;
}

GdnArgs make_args(const lt2_gdn_desc *d, const void *q, const void *k, const void *v, const float *alpha,
                  const float *beta, const float *state_in, void *out, float *state_out, void *ws) {
    GdnArgs a;
    a.B = d->B; a.L = d->L; a.H = d->H; a.dk = d->d_k; a.dv = d->d_v; a.chunk = d->chunk;
    a.qkv_bf16 = d->qkv_dtype == LT2_BF16;
    a.out_bf16 = d->out_dtype == LT2_BF16;
    a.channel = d->gate == LT2_GATE_CHANNEL;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
    a.state_in = state_in; a.out = out; a.state_out = state_out; a.ws = ws;
    return a;
}

size_t prefill_ws(const lt2_gdn_desc *d) {
    if (d->gate == LT2_GATE_CHANNEL)
        return prefill_channel_ws_bytes(d->B, d->L, d->H, d->d_k, d->chunk, d->qkv_dtype == LT2_BF16);
    return prefill_head_ws_bytes(d->B, d->L, d->H, d->chunk);
}

lt2_status hip_status(hipError_t e) { return e == hipSuccess ? LT2_OK : LT2_ERR_HIP; }

}  // namespace

extern "C" {

const char *lt2_status_string(int32_t status) {
    switch (status) {
        case LT2_OK: return "ok";
        case LT2_ERR_NULL: return "required pointer is NULL";
        case LT2_ERR_SHAPE: return "invalid or inconsistent shape";
        case LT2_ERR_DTYPE: return "unknown element type";
        case LT2_ERR_UNSUPPORTED: return "unsupported configuration (head size, chunk or gate)";
        case LT2_ERR_WORKSPACE: return "workspace missing or too small";
        case LT2_ERR_ALIGN: return "pointer not aligned for vector access";
        case LT2_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t lt2_gdn_prefill_workspace_size(const lt2_gdn_desc *desc) {
    if (check_desc(desc, false) != LT2_OK) return 0;
    if (desc->B == 0 || desc->L == 0) return 0;
    return prefill_ws(desc);
}

}  // extern "C"

namespace {

// Shared validation and dispatch of lt2_gdn_prefill and its two phases.
lt2_status prefill_call(int phase, const lt2_gdn_desc *desc, const void *q, const void *k, const void *v,
                        const float *alpha, const float *beta, const float *state_in, void *out,
                        float *state_out, void *ws, size_t ws_bytes, void *stream) {
    lt2_status st = check_desc(desc, false);
    if (st != LT2_OK) return st;
    const bool work = desc->B > 0 && desc->L > 0;
    if (work && (!q || !k)) return LT2_ERR_NULL;
    if (work && (phase & PHASE_PREPARE) && (!alpha || !beta)) return LT2_ERR_NULL;
    if (work && (phase & PHASE_SCAN) && (!v || !out)) return LT2_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(state_in, 16) || !aligned(state_out, 16) || !aligned(alpha, 4) || !aligned(beta, 4))
        return LT2_ERR_ALIGN;
    const size_t need = work ? prefill_ws(desc) : 0;
    if (need > 0 && (!ws || ws_bytes < need)) return LT2_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 16)) return LT2_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (desc->B == 0) return LT2_OK;
    if (desc->L == 0) {
        if (!(phase & PHASE_SCAN) || !state_out) return LT2_OK;
        const size_t n = (size_t)desc->B * desc->H * desc->d_k * desc->d_v;
        return hip_status(launch_state_init(state_out, state_in, n, s));
    }
    GdnArgs a = make_args(desc, q, k, v, alpha, beta, state_in, out, state_out, ws);
    return hip_status(a.channel ? launch_prefill_channel(a, phase, s) : launch_prefill_head(a, phase, s));
}

}  // namespace

extern "C" {

lt2_status lt2_gdn_prefill(const lt2_gdn_desc *desc, const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta, const float *state_in, void *out,
                           float *state_out, void *ws, size_t ws_bytes, void *stream) {
    return prefill_call(PHASE_ALL, desc, q, k, v, alpha, beta, state_in, out, state_out, ws, ws_bytes, stream);
}

lt2_status lt2_gdn_prefill_prepare(const lt2_gdn_desc *desc, const void *q, const void *k, const float *alpha,
                                   const float *beta, void *ws, size_t ws_bytes, void *stream) {
    return prefill_call(PHASE_PREPARE, desc, q, k, nullptr, alpha, beta, nullptr, nullptr, nullptr, ws, ws_bytes,
                        stream);
}

lt2_status lt2_gdn_prefill_scan(const lt2_gdn_desc *desc, const void *q, const void *k, const void *v,
                                const float *state_in, void *out, float *state_out, const void *ws,
                                size_t ws_bytes, void *stream) {
    return prefill_call(PHASE_SCAN, desc, q, k, v, nullptr, nullptr, state_in, out, state_out, (void *)ws, ws_bytes,
                        stream);
}

lt2_status lt2_gdn_decode_step(const lt2_gdn_desc *desc, const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta, float *state, void *out,
                               void *stream) {
    lt2_status st = check_desc(desc, true);
    if (st != LT2_OK) return st;
    if (desc->B > 0 && (!q || !k || !v || !alpha || !beta || !state || !out)) return LT2_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(state, 16) ||
        !aligned(alpha, 4) || !aligned(beta, 4))
        return LT2_ERR_ALIGN;
    if (desc->B == 0) return LT2_OK;
    GdnArgs a = make_args(desc, q, k, v, alpha, beta, state, out, state, nullptr);
    return hip_status(launch_decode(a, (hipStream_t)stream));
}

size_t lt2_gdn_backward_workspace_size(const lt2_gdn_desc *desc) {
    if (check_desc(desc, false) != LT2_OK) return 0;
    if (desc->B == 0 || desc->L == 0) return 0;
    return desc->gate == LT2_GATE_CHANNEL ? kda_bwd_ws_bytes(desc->B, desc->L, desc->H, desc->d_k)
                                          : gdn_bwd_ws_bytes(desc->B, desc->L, desc->H, desc->d_k);
}

lt2_status lt2_gdn_backward(const lt2_gdn_desc *desc, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const float *state_in, const void *d_out,
                            const float *d_state_out, float *dq, float *dk, float *dv, float *dlog_alpha,
                            float *dbeta, float *d_state_in, void *ws, size_t ws_bytes, void *stream) {
    lt2_status st = check_desc(desc, false);
    if (st != LT2_OK) return st;
    const bool channel = desc->gate == LT2_GATE_CHANNEL;
    const bool work = desc->B > 0 && desc->L > 0;
    if (work && (!q || !k || !v || !alpha || !beta || !d_out || !dq || !dk || !dv || !dlog_alpha || !dbeta))
        return LT2_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_out, 16) || !aligned(dq, 16) ||
        !aligned(dk, 16) || !aligned(dv, 16) || !aligned(state_in, 16) || !aligned(d_state_out, 16) ||
        !aligned(d_state_in, 16) || !aligned(alpha, channel ? 16 : 4) || !aligned(beta, 4) ||
        !aligned(dlog_alpha, 4) || !aligned(dbeta, 4))
        return LT2_ERR_ALIGN;
    const size_t need = !work ? 0
                        : channel ? kda_bwd_ws_bytes(desc->B, desc->L, desc->H, desc->d_k)
                                  : gdn_bwd_ws_bytes(desc->B, desc->L, desc->H, desc->d_k);
    if (need > 0 && (!ws || ws_bytes < need)) return LT2_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 16)) return LT2_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (desc->B == 0) return LT2_OK;
    if (desc->L == 0) {
        // no tokens: the state passes through unchanged
        if (!d_state_in) return LT2_OK;
        const size_t n = (size_t)desc->B * desc->H * desc->d_k * desc->d_v;
        return hip_status(launch_state_init(d_state_in, d_state_out, n, s));
    }
    GdnBwdArgs a{};
    a.B = desc->B; a.L = desc->L; a.H = desc->H; a.d = desc->d_k;
    a.qkv_bf16 = desc->qkv_dtype == LT2_BF16; a.dout_bf16 = desc->out_dtype == LT2_BF16;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.state_in = state_in; a.dout = d_out;
    a.dstate_out = d_state_out; a.dq = dq; a.dk = dk; a.dv = dv; a.dlog_alpha = dlog_alpha; a.dbeta = dbeta;
    a.dstate_in = d_state_in; a.ws = ws;
    return hip_status(channel ? launch_kda_bwd(a, s) : launch_gdn_bwd(a, s));
}

lt2_status lt2_swa_prefill(const lt2_swa_desc *desc, const void *q, const void *k, const void *v, void *out,
                           void *stream) {
    if (!desc) return LT2_ERR_NULL;
    if (desc->B < 0 || desc->L < 0 || desc->H <= 0 || desc->d <= 0 || desc->window < 1) return LT2_ERR_SHAPE;
    if ((desc->qkv_dtype != LT2_F32 && desc->qkv_dtype != LT2_BF16) ||
        (desc->out_dtype != LT2_F32 && desc->out_dtype != LT2_BF16))
        return LT2_ERR_DTYPE;
    if (desc->qkv_dtype != LT2_BF16 || (desc->d != 64 && desc->d != 128)) return LT2_ERR_UNSUPPORTED;
    // one workgroup per (b, h, 128 queries): the grid must fit its 31-bit limit
    if ((int64_t)desc->B * desc->H * (((int64_t)desc->L + 127) / 128) > 0x7fffffffLL) return LT2_ERR_SHAPE;
    // key and value tiles are addressed with 32-bit byte offsets within one sequence
    if ((int64_t)desc->L * desc->H * desc->d * 2 > 0x7fffffffLL) return LT2_ERR_SHAPE;
    const bool work = desc->B > 0 && desc->L > 0;
    if (work && (!q || !k || !v || !out)) return LT2_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return LT2_ERR_ALIGN;
    if (!work) return LT2_OK;
    SwaArgs a;
    a.B = desc->B; a.L = desc->L; a.H = desc->H; a.d = desc->d; a.window = desc->window;
    a.out_bf16 = desc->out_dtype == LT2_BF16;
    a.q = q; a.k = k; a.v = v; a.out = out;
    return hip_status(launch_swa(a, (hipStream_t)stream));
}

lt2_status lt2_swa_decode_step(const lt2_swa_desc *desc, const void *q, const void *k, const void *v,
                               void *k_cache, void *v_cache, const int32_t *pos, void *out, void *stream) {
    if (!desc) return LT2_ERR_NULL;
    if (desc->B < 0 || desc->L != 1 || desc->H <= 0 || desc->d <= 0 || desc->window < 1) return LT2_ERR_SHAPE;
    if ((desc->qkv_dtype != LT2_F32 && desc->qkv_dtype != LT2_BF16) ||
        (desc->out_dtype != LT2_F32 && desc->out_dtype != LT2_BF16))
        return LT2_ERR_DTYPE;
    if (desc->qkv_dtype != LT2_BF16 || (desc->d != 64 && desc->d != 128)) return LT2_ERR_UNSUPPORTED;
    // one workgroup per (b, h): the grid must fit its 31-bit limit
    if ((int64_t)desc->B * desc->H > 0x7fffffffLL) return LT2_ERR_SHAPE;
    if (desc->B > 0 && (!q || !k || !v || !k_cache || !v_cache || !pos || !out)) return LT2_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(out, 16) || !aligned(pos, 4))
        return LT2_ERR_ALIGN;
    if (desc->B == 0) return LT2_OK;
    // the rings are distinct buffers (the kernel writes one slot of each and reads the others)
    const size_t ring_bytes = (size_t)desc->B * desc->H * desc->window * desc->d * 2;
    const uintptr_t kb = (uintptr_t)k_cache, vb = (uintptr_t)v_cache;
    if (kb < vb + ring_bytes && vb < kb + ring_bytes) return LT2_ERR_SHAPE;
    SwaDecodeArgs a;
    a.B = desc->B; a.H = desc->H; a.d = desc->d; a.window = desc->window;
    a.out_bf16 = desc->out_dtype == LT2_BF16;
    a.q = q; a.k = k; a.v = v; a.k_cache = k_cache; a.v_cache = v_cache; a.pos = pos; a.out = out;
    return hip_status(launch_swa_decode(a, (hipStream_t)stream));
}

lt2_status lt2_hbm_copy(void *dst, const void *src, size_t bytes, void *stream) {
    if (bytes == 0) return LT2_OK;
    if (!dst || !src) return LT2_ERR_NULL;
    if (bytes % 16 != 0) return LT2_ERR_SHAPE;
    if (!aligned(dst, 16) || !aligned(src, 16)) return LT2_ERR_ALIGN;
    return hip_status(launch_copy(dst, src, bytes, (hipStream_t)stream));
}

lt2_status lt2_hbm_probe(void *dst, const void *src, size_t bytes, int32_t mode, int32_t blocks, int32_t unroll,
                         void *stream) {
    if (mode != LT2_PROBE_COPY && mode != LT2_PROBE_READ && mode != LT2_PROBE_WRITE && mode != LT2_PROBE_TILE_COPY)
        return LT2_ERR_UNSUPPORTED;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16) return LT2_ERR_UNSUPPORTED;
    if (bytes % 16 != 0 || blocks < 0 || blocks > 16777215) return LT2_ERR_SHAPE;
    if (bytes == 0) return LT2_OK;
    if (!dst || (mode != LT2_PROBE_WRITE && !src)) return LT2_ERR_NULL;
    if (!aligned(dst, 16) || !aligned(src, 16)) return LT2_ERR_ALIGN;
    return hip_status(launch_probe(dst, src, bytes, mode, (unsigned)blocks, unroll, (hipStream_t)stream));
}

}  // extern "C"

namespace {

lt2_status check_loop(const lt2_loop_desc *d) {
    if (!d) return LT2_ERR_NULL;
    if (d->B < 0 || d->L < 0 || d->T < 0 || d->d_model <= 0 || d->H <= 0 || d->d_head <= 0) return LT2_ERR_SHAPE;
    if (d->d_head != 64 && d->d_head != 128) return LT2_ERR_UNSUPPORTED;
    if (d->chunk != 16 && d->chunk != 32 && d->chunk != 64) return LT2_ERR_UNSUPPORTED;
    if (d->out_gate != 0 && d->out_gate != 1) return LT2_ERR_UNSUPPORTED;
    // GEMM tiles: K-tiles of 64, residual and head blocks whole 128-column tiles
    if (d->d_model % 128 != 0 || ((int64_t)d->H * d->d_head) % 128 != 0) return LT2_ERR_UNSUPPORTED;
    if ((int64_t)d->B * d->L > 0x7fffffffLL || (int64_t)d->H * d->d_head > 65536 || d->H > 65535 || d->B > 65535)
        return LT2_ERR_SHAPE;
    if (!launch_fits((int64_t)d->B * d->H, d->L, d->chunk)) return LT2_ERR_SHAPE;
    return LT2_OK;
}

}  // namespace

extern "C" {

size_t lt2_looped_mixer_workspace_size(const lt2_loop_desc *desc) {
    if (check_loop(desc) != LT2_OK) return 0;
    if (desc->B == 0 || desc->L == 0) return 0;
    return loop_layout(desc->B, desc->L, desc->d_model, desc->H, desc->d_head, desc->chunk, desc->out_gate).total;
}

lt2_status lt2_looped_mixer(const lt2_loop_desc *desc, const float *h_in, float *h_out, const void *W_in,
                            const void *W_o, void *ws, size_t ws_bytes, void *stream) {
    lt2_status st = check_loop(desc);
    if (st != LT2_OK) return st;
    const bool work = desc->B > 0 && desc->L > 0;
    if (work && (!h_in || !h_out || !W_in || !W_o)) return LT2_ERR_NULL;
    if (!aligned(h_in, 16) || !aligned(h_out, 16) || !aligned(W_in, 16) || !aligned(W_o, 16)) return LT2_ERR_ALIGN;
    const size_t need =
        work ? loop_layout(desc->B, desc->L, desc->d_model, desc->H, desc->d_head, desc->chunk, desc->out_gate).total : 0;
    if (need > 0 && (!ws || ws_bytes < need)) return LT2_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 256)) return LT2_ERR_ALIGN;
    if (!work) return LT2_OK;
    LoopArgs a;
    a.B = desc->B; a.L = desc->L; a.D = desc->d_model; a.H = desc->H; a.d = desc->d_head; a.T = desc->T;
    a.chunk = desc->chunk; a.gated = desc->out_gate; a.h_in = h_in; a.h_out = h_out;
    a.W_in = static_cast<const uint16_t *>(W_in); a.W_o = static_cast<const uint16_t *>(W_o); a.ws = ws;
    return hip_status(launch_looped(a, (hipStream_t)stream));
}

size_t lt2_looped_decode_workspace_size(const lt2_loop_desc *desc) {
    if (check_loop(desc) != LT2_OK || desc->L != 1) return 0;
    if (desc->B == 0) return 0;
    return loop_decode_layout(desc->B, desc->d_model, desc->H, desc->d_head, desc->out_gate).total;
}

}  // extern "C"

namespace {

// Scratch array of lt2_looped_decode_step_noalloc (its workspace).  In host code
// `scratch` names a host-side stand-in, not device memory: kernels receive the
// device address looked up per device below, never the array's name.
static __device__ __align__(256) unsigned char scratch[LT2_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mutex;
void *scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// Device address of the current device's copy of `scratch` (looked up on the
// first call on each device), or nullptr with the runtime's error in *err.
void *scratch_on_current_device(hipError_t *err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        scratch_ptr[dev] = p;
    }
    *err = hipSuccess;
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

lt2_status lt2_looped_decode_step_noalloc(const lt2_loop_desc *desc, float *h, const void *W_in, const void *W_o,
                                          float *states, void *stream) {
    lt2_status st = check_loop(desc);
    if (st != LT2_OK) return st;
    if (desc->L != 1) return LT2_ERR_SHAPE;
    const bool work = desc->B > 0 && desc->T > 0;
    if (work && (!h || !W_in || !W_o || !states)) return LT2_ERR_NULL;
    if (!aligned(h, 16) || !aligned(W_in, 16) || !aligned(W_o, 16) || !aligned(states, 16)) return LT2_ERR_ALIGN;
    if (!work) return LT2_OK;
    const size_t need = loop_decode_layout(desc->B, desc->d_model, desc->H, desc->d_head, desc->out_gate).total;
    if (need > LT2_NOALLOC_SCRATCH_BYTES) return LT2_ERR_WORKSPACE;
    hipError_t err;
    void *ws = scratch_on_current_device(&err);
    if (!ws) return LT2_ERR_HIP;
    LoopDecodeArgs a;
    a.B = desc->B; a.D = desc->d_model; a.H = desc->H; a.d = desc->d_head; a.T = desc->T;
    a.gated = desc->out_gate; a.h = h; a.W_in = static_cast<const uint16_t *>(W_in);
    a.W_o = static_cast<const uint16_t *>(W_o); a.states = states; a.ws = ws;
    return hip_status(launch_looped_decode(a, (hipStream_t)stream));
}

lt2_status lt2_looped_decode_step(const lt2_loop_desc *desc, float *h, const void *W_in, const void *W_o,
                                  float *states, void *ws, size_t ws_bytes, void *stream) {
    lt2_status st = check_loop(desc);
    if (st != LT2_OK) return st;
    if (desc->L != 1) return LT2_ERR_SHAPE;
    const bool work = desc->B > 0 && desc->T > 0;
    if (work && (!h || !W_in || !W_o || !states)) return LT2_ERR_NULL;
    if (!aligned(h, 16) || !aligned(W_in, 16) || !aligned(W_o, 16) || !aligned(states, 16)) return LT2_ERR_ALIGN;
    const size_t need = work ? loop_decode_layout(desc->B, desc->d_model, desc->H, desc->d_head, desc->out_gate).total : 0;
    if (need > 0 && (!ws || ws_bytes < need)) return LT2_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 256)) return LT2_ERR_ALIGN;
    if (!work) return LT2_OK;
    LoopDecodeArgs a;
    a.B = desc->B; a.D = desc->d_model; a.H = desc->H; a.d = desc->d_head; a.T = desc->T;
    a.gated = desc->out_gate; a.h = h; a.W_in = static_cast<const uint16_t *>(W_in); a.W_o = static_cast<const uint16_t *>(W_o);
    a.states = states; a.ws = ws;
    return hip_status(launch_looped_decode(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

lt2_status check_hybrid(const lt2_hybrid_desc *d) {
    if (!d) return LT2_ERR_NULL;
    lt2_loop_desc ld{d->B, d->L, d->d_model, d->H, d->d_head, d->T, d->chunk, d->out_gate};
    const lt2_status st = check_loop(&ld);
    if (st != LT2_OK) return st;
    if (d->n_layers < 1 || d->n_layers > LT2_MAX_LAYERS) return LT2_ERR_SHAPE;
    bool any_swa = false;
    for (int i = 0; i < d->n_layers; ++i) {
        if (d->kinds[i] != LT2_MIXER_GDN && d->kinds[i] != LT2_MIXER_SWA) return LT2_ERR_UNSUPPORTED;
        any_swa = any_swa || d->kinds[i] == LT2_MIXER_SWA;
    }
    if (any_swa) {
        if (d->window < 1) return LT2_ERR_SHAPE;
        if ((int64_t)d->L * d->H * d->d_head * 2 > 0x7fffffffLL ||
            (int64_t)d->B * d->H * (((int64_t)d->L + 127) / 128) > 0x7fffffffLL)
            return LT2_ERR_SHAPE;
    }
    return LT2_OK;
}

}  // namespace

extern "C" {

size_t lt2_hybrid_mixer_workspace_size(const lt2_hybrid_desc *desc) {
    if (check_hybrid(desc) != LT2_OK) return 0;
    if (desc->B == 0 || desc->L == 0) return 0;
    return loop_layout(desc->B, desc->L, desc->d_model, desc->H, desc->d_head, desc->chunk, desc->out_gate).total;
}

lt2_status lt2_hybrid_mixer(const lt2_hybrid_desc *desc, const float *h_in, float *h_out, const void *const *W_in,
                            const void *const *W_o, void *ws, size_t ws_bytes, void *stream) {
    lt2_status st = check_hybrid(desc);
    if (st != LT2_OK) return st;
    const bool work = desc->B > 0 && desc->L > 0;
    if (work && (!h_in || !h_out || !W_in || !W_o)) return LT2_ERR_NULL;
    if (!aligned(h_in, 16) || !aligned(h_out, 16)) return LT2_ERR_ALIGN;
    if (work)
        for (int i = 0; i < desc->n_layers; ++i) {
            if (!W_in[i] || !W_o[i]) return LT2_ERR_NULL;
            if (!aligned(W_in[i], 16) || !aligned(W_o[i], 16)) return LT2_ERR_ALIGN;
        }
    const size_t need =
        work ? loop_layout(desc->B, desc->L, desc->d_model, desc->H, desc->d_head, desc->chunk, desc->out_gate).total : 0;
    if (need > 0 && (!ws || ws_bytes < need)) return LT2_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 256)) return LT2_ERR_ALIGN;
    if (!work) return LT2_OK;
    HybridArgs a{};
    a.B = desc->B; a.L = desc->L; a.D = desc->d_model; a.H = desc->H; a.d = desc->d_head; a.T = desc->T;
    a.chunk = desc->chunk; a.gated = desc->out_gate; a.window = desc->window; a.n_layers = desc->n_layers;
    for (int i = 0; i < desc->n_layers; ++i) {
        a.kinds[i] = desc->kinds[i];
        a.W_in[i] = static_cast<const uint16_t *>(W_in[i]);
        a.W_o[i] = static_cast<const uint16_t *>(W_o[i]);
    }
    a.h_in = h_in; a.h_out = h_out; a.ws = ws;
    return hip_status(launch_hybrid(a, (hipStream_t)stream));
}

size_t lt2_hybrid_decode_workspace_size(const lt2_hybrid_desc *desc) {
    if (check_hybrid(desc) != LT2_OK || desc->L != 1 || desc->B == 0) return 0;
    return loop_decode_layout(desc->B, desc->d_model, desc->H, desc->d_head, desc->out_gate).total;
}

lt2_status lt2_hybrid_decode_step(const lt2_hybrid_desc *desc, float *h, const void *const *W_in,
                                  const void *const *W_o, float *states, void *k_rings, void *v_rings,
                                  const int32_t *pos, void *ws, size_t ws_bytes, void *stream) {
    lt2_status st = check_hybrid(desc);
    if (st != LT2_OK) return st;
    if (desc->L != 1) return LT2_ERR_SHAPE;
    int n_gdn = 0, n_swa = 0;
    for (int i = 0; i < desc->n_layers; ++i) (desc->kinds[i] == LT2_MIXER_GDN ? n_gdn : n_swa)++;
    // one workgroup per (b, h) in the decode kernels
    if ((int64_t)desc->B * desc->H > 0x7fffffffLL) return LT2_ERR_SHAPE;
    const bool work = desc->B > 0 && desc->T > 0;
    if (work && (!h || !W_in || !W_o || !pos || (n_gdn > 0 && !states) || (n_swa > 0 && (!k_rings || !v_rings))))
        return LT2_ERR_NULL;
    if (!aligned(h, 16) || !aligned(states, 16) || !aligned(k_rings, 16) || !aligned(v_rings, 16) || !aligned(pos, 4))
        return LT2_ERR_ALIGN;
    if (work)
        for (int i = 0; i < desc->n_layers; ++i) {
            if (!W_in[i] || !W_o[i]) return LT2_ERR_NULL;
            if (!aligned(W_in[i], 16) || !aligned(W_o[i], 16)) return LT2_ERR_ALIGN;
        }
    const size_t need = work ? loop_decode_layout(desc->B, desc->d_model, desc->H, desc->d_head, desc->out_gate).total : 0;
    if (need > 0 && (!ws || ws_bytes < need)) return LT2_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 256)) return LT2_ERR_ALIGN;
    if (!work) return LT2_OK;
    if (n_swa > 0) {   // distinct key and value rings
        const size_t ring_bytes =
            (size_t)desc->T * n_swa * desc->B * desc->H * desc->window * desc->d_head * 2;
        const uintptr_t kb = (uintptr_t)k_rings, vb = (uintptr_t)v_rings;
        if (kb < vb + ring_bytes && vb < kb + ring_bytes) return LT2_ERR_SHAPE;
    }
    HybridDecodeArgs a{};
    a.B = desc->B; a.D = desc->d_model; a.H = desc->H; a.d = desc->d_head; a.T = desc->T;
    a.gated = desc->out_gate; a.window = desc->window; a.n_layers = desc->n_layers;
    for (int i = 0; i < desc->n_layers; ++i) {
        a.kinds[i] = desc->kinds[i];
        a.W_in[i] = static_cast<const uint16_t *>(W_in[i]);
        a.W_o[i] = static_cast<const uint16_t *>(W_o[i]);
    }
    a.h = h; a.states = states; a.k_rings = static_cast<uint16_t *>(k_rings);
    a.v_rings = static_cast<uint16_t *>(v_rings); a.pos = pos; a.ws = ws;
    return hip_status(launch_hybrid_decode(a, (hipStream_t)stream));
}

}  // extern "C"
