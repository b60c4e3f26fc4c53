/*
 * lt2.h -- C ABI of liblt2.so, the MI355X (gfx950) gated-delta mixer of LT2
 * (Linear-Time Looped Transformers).
 *
 * The operation (LT2 explainer, paithon.it, section "Sostituire il motore",
 * the state-update equation):
 *
 *     S_t = Diag(alpha_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                     (read-out after the update, no scale)
 *
 * per (batch, head) unit, with an fp32 d_k x d_v state.  alpha_t is one value
 * per head (GDN, "scalar gate") or one value per key channel (KDA form,
 * "channel gate"); Diag(alpha_t) scales the rows of the state, after the
 * erase, and the write beta_t k_t v_t^T is not decayed.  The looped driver
 * applies one shared-weight block T times (same page, section "Profondita
 * presa in prestito", first equation).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; it only enqueues kernels on
 *    `stream` (a hipStream_t passed as void*, NULL = the null stream).
 *  - Every call validates all arguments before enqueueing anything.  On any
 *    error nothing is launched and no output is touched.  A launch failure
 *    reported by the HIP runtime maps to LT2_ERR_HIP.
 *  - Row-major layouts, innermost dimension contiguous, no padding:
 *        q, k      [B, L, H, d_k]          token-major
 *        v, out    [B, L, H, d_v]
 *        beta      [B, L, H]    fp32, in [0, 1]
 *        alpha     [B, L, H]    fp32 (scalar gate) or [B, L, H, d_k] (channel
 *                  gate), in [0, 1]; alpha = 0 is allowed (log alpha is
 *                  clamped at -80 inside, a factor below 2e-35)
 *        state     [B, H, d_k, d_v] fp32
 *  - q and k are used exactly as given: no normalisation inside the mixer
 *    (the looped driver normalises its own projections).
 *  - Pointers to q, k, v, out and states must be 16-byte aligned, alpha and
 *    beta 4-byte aligned (LT2_ERR_ALIGN otherwise).
 *  - Supported sizes: d_k == d_v in {64, 128}; chunk in {16, 32, 64} (prefill);
 *    any L >= 0 (a ragged last chunk is masked); B >= 0, H >= 1.
 *  - The library is stateless and re-entrant; calls on one stream run in order.
 */
#ifndef LT2_H
#define LT2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lt2_status {
    LT2_OK = 0,
    LT2_ERR_NULL = 1,        /* a required pointer is NULL */
    LT2_ERR_SHAPE = 2,       /* negative or inconsistent sizes */
    LT2_ERR_DTYPE = 3,       /* unknown element type */
    LT2_ERR_UNSUPPORTED = 4, /* valid but not built: head size, chunk, gate */
    LT2_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
    LT2_ERR_ALIGN = 6,       /* pointer misaligned for its vector loads */
    LT2_ERR_HIP = 7          /* the HIP runtime reported a launch error */
} lt2_status;

typedef enum lt2_dtype { LT2_F32 = 0, LT2_BF16 = 1 } lt2_dtype;

typedef enum lt2_gate {
    LT2_GATE_HEAD = 0,    /* alpha [B, L, H]: one decay per head and token (GDN) */
    LT2_GATE_CHANNEL = 1  /* alpha [B, L, H, d_k]: one decay per key channel (KDA) */
} lt2_gate;

/* Shape and types of one gated-delta call. */
typedef struct lt2_gdn_desc {
    int32_t B, L, H;     /* batch, tokens, heads */
    int32_t d_k, d_v;    /* key and value head size */
    int32_t chunk;       /* prefill chunk length C (16, 32 or 64); ignored by decode */
    int32_t qkv_dtype;   /* lt2_dtype of q, k and v */
    int32_t out_dtype;   /* lt2_dtype of out */
    int32_t gate;        /* lt2_gate */
} lt2_gdn_desc;

/* Shape of the looped LT2-linear block. */
typedef struct lt2_loop_desc {
    int32_t B, L;        /* sequences, tokens per sequence */
    int32_t d_model;     /* residual width D */
    int32_t H, d_head;   /* heads and head size (d_k = d_v = d_head) */
    int32_t T;           /* loops with shared weights */
    int32_t chunk;       /* prefill chunk length of the mixer */
    int32_t out_gate;    /* 1: sigmoid output gate inside the loop (W_g rows in W_in), 0: none */
} lt2_loop_desc;

/* Human-readable name of a status code (static string, never NULL); any value
 * outside lt2_status gives "unknown status". */
const char *lt2_status_string(int32_t status);

/*
 * Workspace bytes lt2_gdn_prefill needs for `desc` (0 if none).  Returns 0 for
 * an invalid descriptor (lt2_gdn_prefill then reports the error).
 */
size_t lt2_gdn_prefill_workspace_size(const lt2_gdn_desc *desc);

/*
 * Chunked prefill: run the recurrence over all L tokens of every (b, h) unit.
 *   q, k, v     inputs, element type desc->qkv_dtype, layouts above
 *   alpha, beta fp32 gates
 *   state_in    initial state [B,H,d_k,d_v] fp32, or NULL for S_0 = 0
 *   out         o_t for every token, element type desc->out_dtype
 *   state_out   final state S_L, or NULL; may equal state_in (in-place)
 *   ws/ws_bytes device workspace of at least lt2_gdn_prefill_workspace_size()
 * Inside each chunk of C tokens the state-independent part (the WY/UT factors
 * of the chunk) is formed in parallel over chunks; the state is then carried
 * across chunks in fp32, one chunk after the other per unit.
 */
lt2_status lt2_gdn_prefill(const lt2_gdn_desc *desc, const void *q, const void *k,
                           const void *v, const float *alpha, const float *beta,
                           const float *state_in, void *out, float *state_out,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * The two phases of lt2_gdn_prefill, for callers that schedule them apart
 * (e.g. overlap the prepare phase of the next batch with the scan of this one,
 * or time them separately).  lt2_gdn_prefill(...) is exactly
 * lt2_gdn_prefill_prepare(...) followed by lt2_gdn_prefill_scan(...) on one
 * stream with the same descriptor and workspace.
 *   prepare: reads q, k, alpha, beta; writes the state-independent factors
 *            of every chunk into ws (chunk-parallel).
 *   scan:    reads q, k, v and the factors in ws; carries the fp32 state
 *            across the chunks of every unit in order; writes out, state_out.
 * Arguments, layouts and errors as for lt2_gdn_prefill; the workspace contents
 * between the two calls are private to the library.
 */
lt2_status lt2_gdn_prefill_prepare(const lt2_gdn_desc *desc, const void *q, const void *k,
                                   const float *alpha, const float *beta, void *ws,
                                   size_t ws_bytes, void *stream);
lt2_status lt2_gdn_prefill_scan(const lt2_gdn_desc *desc, const void *q, const void *k,
                                const void *v, const float *state_in, void *out,
                                float *state_out, const void *ws, size_t ws_bytes,
                                void *stream);

/*
 * One decode token (desc->L must be 1) for every (b, h) unit, state updated in
 * place.  q, k [B,H,d_k], v, out [B,H,d_v] (element types from desc),
 * alpha [B,H] or [B,H,d_k], beta [B,H] fp32, state [B,H,d_k,d_v] fp32.
 * The state is read once and written once.  No workspace.
 */
lt2_status lt2_gdn_decode_step(const lt2_gdn_desc *desc, const void *q, const void *k,
                               const void *v, const float *alpha, const float *beta,
                               float *state, void *out, void *stream);

/*
 * Workspace bytes lt2_looped_mixer needs (0 for an invalid descriptor).
 */
size_t lt2_looped_mixer_workspace_size(const lt2_loop_desc *desc);

/*
 * T loops of the LT2-linear block with shared weights, fresh zero state in
 * every loop:
 *     z = bf16(h) W_in^T                      [B*L, 3*H*d + 2*H] (+ H*d gated)
 *     q, k = per-head L2 normalisation of z's first two H*d blocks
 *            (x / max(||x||_2, 1e-6)), v = third block
 *     beta = sigmoid(z_beta), alpha = exp(-softplus(z_alpha))  (one per head)
 *     o = gated-delta prefill(q, k, v, alpha, beta; S_0 = 0)    bf16
 *     desc->out_gate: o = o * sigmoid(z_g), z_g the fourth H*d block (the
 *            sigmoid output gate the LT2 explainer places inside the loop)
 *     h = h + o W_o^T                          fp32 residual stream
 *   h_in, h_out   [B, L, d_model] fp32 (may be the same buffer)
 *   W_in          [3*H*d + 2*H, d_model] bf16, rows W_q, W_k, W_v, W_beta, W_alpha;
 *                 with out_gate [4*H*d + 2*H, d_model], rows W_q, W_k, W_v, W_g,
 *                 W_beta, W_alpha
 *   W_o           [d_model, H*d] bf16
 * Weight layout: every weight is stored [d_out, d_in] (row i holds the
 * weights of output feature i) and applied as x W^T, so both operands of each
 * product run contiguously along the reduction dimension.  This departs from
 * the row-vector convention x W with W stored [d_in, d_out]: a caller holding
 * weights that way passes their transposes (W_in = [W_q W_k W_v W_beta
 * W_alpha]^T).  The same layout holds for lt2_looped_decode_step and
 * lt2_hybrid_mixer.
 * Requirements: d_model % 128 == 0, H*d % 128 == 0, d in {64, 128}.
 */
lt2_status lt2_looped_mixer(const lt2_loop_desc *desc, const float *h_in, float *h_out,
                            const void *W_in, const void *W_o, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * Workspace bytes lt2_looped_decode_step needs (0 for an invalid descriptor,
 * which includes desc->L != 1).
 */
size_t lt2_looped_decode_workspace_size(const lt2_loop_desc *desc);

/*
 * One decode token of the looped LT2-linear block for each of B sequences
 * (the loop equation of the LT2 explainer, paithon.it, "Profondita presa in
 * prestito", with the mixer in its recurrent form of "Sostituire il motore"):
 * the T loops of lt2_looped_mixer applied to the new token, loop t carrying
 * its own state across calls.  desc->L must be 1.
 *   h        [B, d_model] fp32, the token's residual stream, updated in place
 *   W_in     as for lt2_looped_mixer (with W_g rows when desc->out_gate)
 *   W_o      [d_model, H*d] bf16
 *   states   [T, B, H, d_head, d_head] fp32, loop t's state of every (b, h),
 *            updated in place; zero before a sequence's first token
 *   ws       at least lt2_looped_decode_workspace_size(desc) bytes, 256-aligned
 * Each state is read once and written once per loop.  Because every loop's
 * mixer is causal, calling this on tokens 1..L of a sequence from zero states
 * yields, token by token, the h that lt2_looped_mixer gives for the sequence.
 * Errors: LT2_ERR_SHAPE for L != 1; otherwise as lt2_looped_mixer.
 */
lt2_status lt2_looped_decode_step(const lt2_loop_desc *desc, float *h, const void *W_in,
                                  const void *W_o, float *states, void *ws, size_t ws_bytes,
                                  void *stream);

/*
 * Scratch capacity of lt2_looped_decode_step_noalloc: a fixed device array of
 * this many bytes, one per GPU the library runs on, held until the process
 * ends.
 */
#define LT2_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * lt2_looped_decode_step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * lt2_looped_decode_step with its workspace replaced by the library's
 * fixed-size scratch array on the current device: the call allocates and frees
 * nothing and uses no workspace argument.  Every buffer in the scratch array is
 * written before it is read within one call, so nothing needs clearing.
 * Limit: lt2_looped_decode_workspace_size(desc) <= LT2_NOALLOC_SCRATCH_BYTES
 * (32 MiB: e.g. up to 1024 sequences at d_model 2048 with 16 heads of 128, with
 * the output gate), else LT2_ERR_WORKSPACE and nothing is launched.
 * Concurrency: all calls on one GPU share its scratch array, so calls that may
 * overlap on one GPU (different streams, or host threads without ordering)
 * race; serialise them (one stream) or use lt2_looped_decode_step.  The first
 * call on a device looks up that device's copy of the array
 * (LT2_ERR_HIP if the runtime cannot).
 */
lt2_status lt2_looped_decode_step_noalloc(const lt2_loop_desc *desc, float *h, const void *W_in,
                                          const void *W_o, float *states, void *stream);

/*
 * Workspace bytes lt2_gdn_backward needs (0 for an invalid descriptor).
 */
size_t lt2_gdn_backward_workspace_size(const lt2_gdn_desc *desc);

/*
 * Backward pass of lt2_gdn_prefill: the gradients of a loss whose cotangents
 * are d_out for the outputs o and d_state_out for the final state, through the
 * state-update equation of the LT2 explainer (paithon.it, "Sostituire il
 * motore") with o_t = S_t^T q_t, for either gate.
 *   q, k, v, alpha, beta, state_in   the forward call's inputs (state_in NULL = 0)
 *   d_out        [B, L, H, d_v] of desc->out_dtype
 *   d_state_out  [B, H, d_k, d_v] fp32, or NULL (= 0)
 *   dq, dk       [B, L, H, d_k] fp32      dv  [B, L, H, d_v] fp32
 *   dlog_alpha   the gradient with respect to log alpha_t, alpha's shape:
 *                [B, L, H] (scalar gate) or [B, L, H, d_k] (channel gate), fp32
 *                (finite at alpha = 0; divide by alpha for d/d alpha)
 *   dbeta        [B, L, H] fp32
 *   d_state_in   [B, H, d_k, d_v] fp32, or NULL when not wanted
 *   ws           at least lt2_gdn_backward_workspace_size(desc) bytes, 16-aligned
 * With the channel gate alpha must be 16-byte aligned (read 16 bytes at a time).
 * Arithmetic is fp32 throughout (bf16 inputs are widened exactly).  Scalar
 * gate: the chunk form on the matrix cores with chunk 64 whatever desc->chunk
 * holds.  Channel gate: the token adjoint on the vector ALUs, with the state
 * checkpointed every 16 tokens in the workspace (d_k^2 * 4 bytes per 16 tokens
 * per unit, plus d_k/16 partial sums of the row gradients).  The result does
 * not depend on desc->chunk.  Errors as for lt2_gdn_prefill.
 */
lt2_status lt2_gdn_backward(const lt2_gdn_desc *desc, const void *q, const void *k,
                            const void *v, const float *alpha, const float *beta,
                            const float *state_in, const void *d_out, const float *d_state_out,
                            float *dq, float *dk, float *dv, float *dlog_alpha, float *dbeta,
                            float *d_state_in, void *ws, size_t ws_bytes, void *stream);

/* Shape and types of one sliding-window attention call. */
typedef struct lt2_swa_desc {
    int32_t B, L, H;     /* batch, tokens, heads */
    int32_t d;           /* head size (q, k and v) */
    int32_t window;      /* w >= 1: query t attends to keys t-w+1 .. t */
    int32_t qkv_dtype;   /* lt2_dtype of q, k and v (LT2_BF16 is built) */
    int32_t out_dtype;   /* lt2_dtype of out */
} lt2_swa_desc;

/*
 * Causal sliding-window softmax attention, the sparse mixer family of LT2
 * (LT2 explainer, paithon.it, section "Sostituire il motore": each token looks
 * only at a window of the w most recent positions):
 *     o_t = sum_{j=max(0,t-w+1)}^{t} softmax_j(q_t . k_j / sqrt(d)) v_j
 * for every batch entry and head; w >= L gives causal full attention.
 *   q, k, v   [B, L, H, d] bf16, 16-byte aligned, used as given
 *   out       [B, L, H, d] bf16 or fp32 (desc->out_dtype), 16-byte aligned
 * Scores and the softmax are fp32; the probabilities enter the value product
 * as bf16 with fp32 accumulation.  No workspace.
 * Limits: one sequence's q (L * H * d bf16) below 2 GiB.
 * Errors: LT2_ERR_SHAPE for negative sizes, window < 1 or sizes beyond the
 * limits; LT2_ERR_UNSUPPORTED
 * for fp32 q/k/v or d not in {64, 128}; LT2_ERR_NULL / LT2_ERR_ALIGN as usual.
 */
lt2_status lt2_swa_prefill(const lt2_swa_desc *desc, const void *q, const void *k, const void *v,
                           void *out, void *stream);

/*
 * One decode token of the sliding-window mixer (the decode form of
 * lt2_swa_prefill; LT2 explainer, paithon.it, section "Sostituire il motore":
 * each token attends to the w most recent positions, itself included).  For
 * every batch entry b and head, the window is a ring of the last w keys and
 * values: the new token's k and v are written to ring slot pos[b] mod w, then
 *     o = sum_j softmax_j(q . k_j / sqrt(d)) v_j
 * over the filled slots, which hold the tokens max(0, pos[b]-w+1) .. pos[b]
 * (the softmax does not depend on the order of the slots).
 *   desc              B, H, d, window; L must be 1; qkv_dtype LT2_BF16
 *   q, k, v           [B, H, d] bf16, the new token, 16-byte aligned
 *   k_cache, v_cache  [B, H, window, d] bf16, owned by the caller and updated
 *                     in place (slot pos[b] mod window); slots past pos[b] are
 *                     never read while pos[b] < window - 1, so fresh rings need
 *                     no initialisation; two distinct, non-overlapping buffers
 *                     (out must not overlap q, k, v or the rings either)
 *   pos               [B] int32 in device memory: tokens sequence b has already
 *                     seen (the new token's position); negative values are
 *                     taken as 0.  The call does not advance it.
 *   out               [B, H, d] bf16 or fp32 (desc->out_dtype), 16-byte aligned
 * Scores, the softmax and the value sums are fp32.  No workspace.
 * Errors: LT2_ERR_SHAPE for L != 1, negative B, H or d <= 0, window < 1,
 * B * H beyond 2^31 - 1 or overlapping rings; LT2_ERR_DTYPE / LT2_ERR_UNSUPPORTED as for
 * lt2_swa_prefill; LT2_ERR_NULL for a missing pointer when B > 0;
 * LT2_ERR_ALIGN for misaligned buffers (pos: 4 bytes).
 */
lt2_status lt2_swa_decode_step(const lt2_swa_desc *desc, const void *q, const void *k, const void *v,
                               void *k_cache, void *v_cache, const int32_t *pos, void *out, void *stream);

/* Layer kinds of the looped hybrid block. */
#define LT2_MAX_LAYERS 8
typedef enum lt2_mixer_kind {
    LT2_MIXER_GDN = 0,   /* gated-delta layer, as in lt2_looped_mixer */
    LT2_MIXER_SWA = 1    /* sliding-window attention layer */
} lt2_mixer_kind;

/* Shape of the looped hybrid block: n_layers layers applied in order, T times. */
typedef struct lt2_hybrid_desc {
    int32_t B, L, d_model, H, d_head, T, chunk, out_gate;   /* as lt2_loop_desc */
    int32_t window;                      /* window w of the SWA layers (>= 1) */
    int32_t n_layers;                    /* 1 .. LT2_MAX_LAYERS */
    int32_t kinds[LT2_MAX_LAYERS];       /* lt2_mixer_kind of each layer */
} lt2_hybrid_desc;

/*
 * Workspace bytes lt2_hybrid_mixer needs (0 for an invalid descriptor); the
 * same as lt2_looped_mixer's for the same sizes (layers share the buffers).
 */
size_t lt2_hybrid_mixer_workspace_size(const lt2_hybrid_desc *desc);

/*
 * The looped hybrid block: the LT2 summary page's hybrid strategies interleave
 * linear (gated-delta) and sparse (window) mixers across depth and loops; here
 * the shared block is a stack of desc->n_layers layers run in order, each with
 * its own weights, and the block is applied T times with the same weights.
 *   gated-delta layer i: exactly one loop of lt2_looped_mixer with W_in[i], W_o[i]
 *   window layer i:      z = bf16(h) W_in[i]^T, q, k, v = z's first three H*d
 *                        blocks (no normalisation), o = lt2_swa_prefill(q, k, v;
 *                        desc->window) in bf16, with out_gate o = o * sigmoid(z_g)
 *                        (z_g the fourth block), h = h + o W_o[i]^T
 *   W_in, W_o  host arrays of n_layers device pointers (bf16):
 *              gated-delta layer: W_in [3*H*d + 2*H (+ H*d), d_model] as for
 *              lt2_looped_mixer; window layer: W_in [3*H*d (+ H*d), d_model],
 *              rows W_q, W_k, W_v (, W_g); W_o [d_model, H*d] for both
 *   h_in, h_out [B, L, d_model] fp32 (may be the same buffer)
 * A block of one gated-delta layer is lt2_looped_mixer.  Requirements as for
 * lt2_looped_mixer, and for window layers those of lt2_swa_prefill.
 * Errors: LT2_ERR_SHAPE for n_layers outside 1..LT2_MAX_LAYERS or window < 1
 * with a window layer; LT2_ERR_UNSUPPORTED for an unknown layer kind; otherwise
 * as lt2_looped_mixer.
 */
lt2_status lt2_hybrid_mixer(const lt2_hybrid_desc *desc, const float *h_in, float *h_out,
                            const void *const *W_in, const void *const *W_o, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * Looped hybrid decode: one new token per sequence through the T loops of the
 * shared layer stack of lt2_hybrid_mixer (LT2 summary page, hybrid strategies
 * across depth and iterations; the mixers' decode forms as in
 * lt2_gdn_decode_step and lt2_swa_decode_step).  Loop tau's layer l carries its
 * own recurrent state (gated-delta layers) or ring of the last w keys and
 * values (window layers) across calls; by causality, token-by-token calls from
 * zero states and empty rings reproduce lt2_hybrid_mixer on the whole sequence.
 *   desc      as lt2_hybrid_mixer with L = 1 (chunk is not used)
 *   h         [B, d_model] fp32, the token's residual stream, updated in place
 *   W_in, W_o host arrays of n_layers device pointers, layouts as
 *             lt2_hybrid_mixer
 *   states    [T, n_gdn, B, H, d_head, d_head] fp32, in place (n_gdn = number of
 *             gated-delta layers, indexed in stack order); may be NULL if none
 *   k_rings, v_rings  [T, n_swa, B, H, window, d_head] bf16, in place (n_swa =
 *             number of window layers), two non-overlapping buffers; slot
 *             pos[b] mod window is written
 *   pos       [B] int32 in device memory: tokens sequence b has already seen;
 *             not advanced by the call
 *   ws        lt2_hybrid_decode_workspace_size(desc) bytes, 256-byte aligned
 * Errors: as lt2_hybrid_mixer; LT2_ERR_SHAPE for L != 1 or overlapping rings.
 */
size_t lt2_hybrid_decode_workspace_size(const lt2_hybrid_desc *desc);
lt2_status lt2_hybrid_decode_step(const lt2_hybrid_desc *desc, float *h, const void *const *W_in,
                                  const void *const *W_o, float *states, void *k_rings, void *v_rings,
                                  const int32_t *pos, void *ws, size_t ws_bytes, void *stream);

/*
 * Bandwidth probe: copy `bytes` (a multiple of 16) from src to dst with one
 * streaming kernel.  Used to measure the achievable HBM bandwidth.
 */
lt2_status lt2_hbm_copy(void *dst, const void *src, size_t bytes, void *stream);

/* Access patterns of lt2_hbm_probe. */
typedef enum lt2_probe_mode {
    LT2_PROBE_COPY = 0,   /* read src, write dst */
    LT2_PROBE_READ = 1,   /* read src only (dst is not written in practice) */
    LT2_PROBE_WRITE = 2,  /* write dst only (src unused, may be NULL) */
    LT2_PROBE_TILE_COPY = 3   /* read src, write dst, each workgroup copying contiguous
                                 tiles of 256 x unroll 16-byte elements, every load of a
                                 tile issued before its stores */
} lt2_probe_mode;

/*
 * Bandwidth probe with a chosen launch shape, for finding the achievable HBM
 * bandwidth of each access pattern (the best over shapes is the measured
 * ceiling the memory-bound kernels are compared with).  One streaming kernel
 * of `blocks` workgroups of 256 lanes (0 = the default of 16 per compute unit
 * of a 256-CU device), each lane keeping `unroll` 16-byte loads (or stores) in
 * flight; grid-stride over single elements, or over whole tiles for
 * LT2_PROBE_TILE_COPY.
 *   dst, src   device buffers of `bytes` bytes each (a multiple of 16),
 *              16-byte aligned; src may be NULL for LT2_PROBE_WRITE
 *   mode       lt2_probe_mode
 *   blocks     0 .. 16777215     unroll  1, 2, 4, 8 or 16
 * Errors: LT2_ERR_NULL, LT2_ERR_ALIGN as usual; LT2_ERR_SHAPE for a size not a
 * multiple of 16 or blocks out of range; LT2_ERR_UNSUPPORTED for another mode
 * or unroll.
 */
lt2_status lt2_hbm_probe(void *dst, const void *src, size_t bytes, int32_t mode, int32_t blocks,
                         int32_t unroll, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LT2_H */
