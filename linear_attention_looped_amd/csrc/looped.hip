// looped.hip -- the looped LT2-linear block: T applications of one shared-weight
// block (LT2 explainer, paithon.it, "Profondita presa in prestito", first
// equation), each a gated-delta mixer with fresh zero state:
//   xb = bf16(h)                                    (cast kernel, first loop only)
//   [q|k|v|beta|alpha] = xb W_in^T  + per-head L2 norm and gate transforms (GEMM)
//   o = gated-delta prefill(q, k, v, alpha, beta; S_0 = 0), bf16
//   optional output gate (the explainer's sigmoid gate inside the loop):
//   o = o * sigmoid(xb W_g^T), one gate per channel, applied where o is stored
//   h += o W_o^T, xb = bf16(h)                      (GEMM with residual epilogue)
// All launches are enqueued on one stream; nothing synchronises in between.
//
// Looped hybrid: the shared block is a fixed stack of layers, each a
// gated-delta mixer as above or a sliding-window attention mixer (the LT2
// summary page's hybrids interleave the two kinds across depth); a window layer
// projects q, k, v (and g) without normalisation and has no gate transforms.
//
// Looped decode: one new token per sequence through the same T loops, loop t
// carrying its own recurrent state across calls (the decode form of the mixer,
// state update equation of "Sostituire il motore"):
//   xb = bf16(h); for t: [q|k|v|beta|alpha] = xb W_in^T (as above);
//   o = decode step on state t; h += o W_o^T, xb = bf16(h)
#include "gemm.h"
#include "internal.h"

namespace lt2 {

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

LoopLayout loop_layout(int B, int L, int D, int H, int d, int chunk, bool gated) {
    LoopLayout w{};
    const size_t M = (size_t)B * L, Hd = (size_t)H * d;
    size_t off = 0;
    w.xb = off; off = align256(off + M * D * 2);
    w.q = off; off = align256(off + M * Hd * 2);
    w.k = off; off = align256(off + M * Hd * 2);
    w.v = off; off = align256(off + M * Hd * 2);
    w.g = off; off = align256(off + (gated ? M * Hd * 2 : 0));
    w.beta = off; off = align256(off + M * H * 4);
    w.alpha = off; off = align256(off + M * H * 4);
    w.o = off; off = align256(off + M * Hd * 2);
    w.prefill = off; off = align256(off + prefill_head_ws_bytes(B, L, H, chunk));
    w.total = off;
    return w;
}

LoopLayout loop_decode_layout(int B, int D, int H, int d, bool gated) {
    LoopLayout w{};
    const size_t M = (size_t)B, Hd = (size_t)H * d;
    size_t off = 0;
    w.xb = off; off = align256(off + M * D * 2);
    w.q = off; off = align256(off + M * Hd * 2);
    w.k = off; off = align256(off + M * Hd * 2);
    w.v = off; off = align256(off + M * Hd * 2);
    w.g = off; off = align256(off + (gated ? M * Hd * 2 : 0));
    w.beta = off; off = align256(off + M * H * 4);
    w.alpha = off; off = align256(off + M * H * 4);
    w.o = off; off = align256(off + M * Hd * 2);
    w.prefill = off;
    w.total = off;
    return w;
}

hipError_t launch_looped_decode(const LoopDecodeArgs &a, hipStream_t s) {
    const int M = a.B, Hd = a.H * a.d, N_in = (a.gated ? 4 : 3) * Hd + 2 * a.H;
    unsigned char *ws = static_cast<unsigned char *>(a.ws);
    const LoopLayout w = loop_decode_layout(a.B, a.D, a.H, a.d, a.gated);
    uint16_t *gt = a.gated ? reinterpret_cast<uint16_t *>(ws + w.g) : nullptr;
    uint16_t *xb = reinterpret_cast<uint16_t *>(ws + w.xb);
    uint16_t *q = reinterpret_cast<uint16_t *>(ws + w.q);
    uint16_t *k = reinterpret_cast<uint16_t *>(ws + w.k);
    uint16_t *v = reinterpret_cast<uint16_t *>(ws + w.v);
    float *beta = reinterpret_cast<float *>(ws + w.beta);
    float *alpha = reinterpret_cast<float *>(ws + w.alpha);
    uint16_t *o = reinterpret_cast<uint16_t *>(ws + w.o);

    hipError_t e = launch_cast_residual(a.h, a.h, xb, (size_t)M * a.D, s);
    if (e != hipSuccess) return e;
    GdnArgs g{};
    g.B = a.B; g.L = 1; g.H = a.H; g.dk = a.d; g.dv = a.d; g.chunk = 64;
    g.qkv_bf16 = 1; g.out_bf16 = 1; g.channel = 0;
    g.q = q; g.k = k; g.v = v; g.alpha = alpha; g.beta = beta; g.out = o; g.gate = gt;
    const size_t state_elems = (size_t)a.B * a.H * a.d * a.d;
    for (int t = 0; t < a.T; ++t) {
        e = launch_gemm_proj(xb, a.W_in, M, N_in, a.D, q, k, v, gt, beta, alpha, a.H, a.d, s);
        if (e != hipSuccess) return e;
        g.state_in = a.states + (size_t)t * state_elems;
        g.state_out = a.states + (size_t)t * state_elems;
        e = launch_decode(g, s);
        if (e != hipSuccess) return e;
        e = launch_gemm_resid(o, a.W_o, M, a.D, Hd, a.h, xb, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_looped(const LoopArgs &a, hipStream_t s) {
    const int M = a.B * a.L, Hd = a.H * a.d, N_in = (a.gated ? 4 : 3) * Hd + 2 * a.H;
    unsigned char *ws = static_cast<unsigned char *>(a.ws);
    const LoopLayout w = loop_layout(a.B, a.L, a.D, a.H, a.d, a.chunk, a.gated);
    uint16_t *gt = a.gated ? reinterpret_cast<uint16_t *>(ws + w.g) : nullptr;
    uint16_t *xb = reinterpret_cast<uint16_t *>(ws + w.xb);
    uint16_t *q = reinterpret_cast<uint16_t *>(ws + w.q);
    uint16_t *k = reinterpret_cast<uint16_t *>(ws + w.k);
    uint16_t *v = reinterpret_cast<uint16_t *>(ws + w.v);
    float *beta = reinterpret_cast<float *>(ws + w.beta);
    float *alpha = reinterpret_cast<float *>(ws + w.alpha);
    uint16_t *o = reinterpret_cast<uint16_t *>(ws + w.o);

    hipError_t e = launch_cast_residual(a.h_in, a.h_out, xb, (size_t)M * a.D, s);
    if (e != hipSuccess) return e;
    GdnArgs g{};
    g.B = a.B; g.L = a.L; g.H = a.H; g.dk = a.d; g.dv = a.d; g.chunk = a.chunk;
    g.qkv_bf16 = 1; g.out_bf16 = 1; g.channel = 0;
    g.q = q; g.k = k; g.v = v; g.alpha = alpha; g.beta = beta;
    g.state_in = nullptr; g.out = o; g.state_out = nullptr; g.ws = ws + w.prefill; g.gate = gt;
    for (int t = 0; t < a.T; ++t) {
        e = launch_gemm_proj(xb, a.W_in, M, N_in, a.D, q, k, v, gt, beta, alpha, a.H, a.d, s);
        if (e != hipSuccess) return e;
        e = launch_prefill_head(g, PHASE_ALL, s);
        if (e != hipSuccess) return e;
        e = launch_gemm_resid(o, a.W_o, M, a.D, Hd, a.h_out, xb, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_hybrid(const HybridArgs &a, hipStream_t s) {
    const int M = a.B * a.L, Hd = a.H * a.d, NR = a.gated ? 4 : 3;
    unsigned char *ws = static_cast<unsigned char *>(a.ws);
    const LoopLayout w = loop_layout(a.B, a.L, a.D, a.H, a.d, a.chunk, a.gated);
    uint16_t *gt = a.gated ? reinterpret_cast<uint16_t *>(ws + w.g) : nullptr;
    uint16_t *xb = reinterpret_cast<uint16_t *>(ws + w.xb);
    uint16_t *q = reinterpret_cast<uint16_t *>(ws + w.q);
    uint16_t *k = reinterpret_cast<uint16_t *>(ws + w.k);
    uint16_t *v = reinterpret_cast<uint16_t *>(ws + w.v);
    float *beta = reinterpret_cast<float *>(ws + w.beta);
    float *alpha = reinterpret_cast<float *>(ws + w.alpha);
    uint16_t *o = reinterpret_cast<uint16_t *>(ws + w.o);

    hipError_t e = launch_cast_residual(a.h_in, a.h_out, xb, (size_t)M * a.D, s);
    if (e != hipSuccess) return e;
    GdnArgs g{};
    g.B = a.B; g.L = a.L; g.H = a.H; g.dk = a.d; g.dv = a.d; g.chunk = a.chunk;
    g.qkv_bf16 = 1; g.out_bf16 = 1; g.channel = 0;
    g.q = q; g.k = k; g.v = v; g.alpha = alpha; g.beta = beta;
    g.state_in = nullptr; g.out = o; g.state_out = nullptr; g.ws = ws + w.prefill; g.gate = gt;
    SwaArgs sw{};
    sw.B = a.B; sw.L = a.L; sw.H = a.H; sw.d = a.d; sw.window = a.window; sw.out_bf16 = 1;
    sw.q = q; sw.k = k; sw.v = v; sw.out = o; sw.gate = gt;
    for (int t = 0; t < a.T; ++t)
        for (int i = 0; i < a.n_layers; ++i) {
            if (a.kinds[i] == 0) {
                e = launch_gemm_proj(xb, a.W_in[i], M, NR * Hd + 2 * a.H, a.D, q, k, v, gt, beta, alpha, a.H, a.d, s);
                if (e == hipSuccess) e = launch_prefill_head(g, PHASE_ALL, s);
            } else {
                e = launch_gemm_proj(xb, a.W_in[i], M, NR * Hd, a.D, q, k, v, gt, nullptr, nullptr, a.H, a.d, s,
                                     false);
                if (e == hipSuccess) e = launch_swa(sw, s);
            }
            if (e == hipSuccess) e = launch_gemm_resid(o, a.W_o[i], M, a.D, Hd, a.h_out, xb, s);
            if (e != hipSuccess) return e;
        }
    return hipSuccess;
}

hipError_t launch_hybrid_decode(const HybridDecodeArgs &a, hipStream_t s) {
    const int M = a.B, Hd = a.H * a.d, NR = a.gated ? 4 : 3;
    unsigned char *ws = static_cast<unsigned char *>(a.ws);
    const LoopLayout w = loop_decode_layout(a.B, a.D, a.H, a.d, a.gated);
    uint16_t *gt = a.gated ? reinterpret_cast<uint16_t *>(ws + w.g) : nullptr;
    uint16_t *xb = reinterpret_cast<uint16_t *>(ws + w.xb);
    uint16_t *q = reinterpret_cast<uint16_t *>(ws + w.q);
    uint16_t *k = reinterpret_cast<uint16_t *>(ws + w.k);
    uint16_t *v = reinterpret_cast<uint16_t *>(ws + w.v);
    float *beta = reinterpret_cast<float *>(ws + w.beta);
    float *alpha = reinterpret_cast<float *>(ws + w.alpha);
    uint16_t *o = reinterpret_cast<uint16_t *>(ws + w.o);
    int n_gdn = 0, n_swa = 0;
    for (int i = 0; i < a.n_layers; ++i) (a.kinds[i] == 0 ? n_gdn : n_swa)++;
    const size_t state_elems = (size_t)a.B * a.H * a.d * a.d;
    const size_t ring_elems = (size_t)a.B * a.H * a.window * a.d;

    hipError_t e = launch_cast_residual(a.h, a.h, xb, (size_t)M * a.D, s);
    if (e != hipSuccess) return e;
    GdnArgs g{};
    g.B = a.B; g.L = 1; g.H = a.H; g.dk = a.d; g.dv = a.d; g.chunk = 64;
    g.qkv_bf16 = 1; g.out_bf16 = 1; g.channel = 0;
    g.q = q; g.k = k; g.v = v; g.alpha = alpha; g.beta = beta; g.out = o; g.gate = gt;
    SwaDecodeArgs sw{};
    sw.B = a.B; sw.H = a.H; sw.d = a.d; sw.window = a.window; sw.out_bf16 = 1;
    sw.q = q; sw.k = k; sw.v = v; sw.pos = a.pos; sw.out = o; sw.gate = gt;
    for (int t = 0; t < a.T; ++t) {
        int gi = 0, si = 0;   // this loop's gated-delta and window layers so far
        for (int i = 0; i < a.n_layers; ++i) {
            if (a.kinds[i] == 0) {
                e = launch_gemm_proj(xb, a.W_in[i], M, NR * Hd + 2 * a.H, a.D, q, k, v, gt, beta, alpha, a.H, a.d, s);
                g.state_in = g.state_out = a.states + ((size_t)t * n_gdn + gi++) * state_elems;
                if (e == hipSuccess) e = launch_decode(g, s);
            } else {
                e = launch_gemm_proj(xb, a.W_in[i], M, NR * Hd, a.D, q, k, v, gt, nullptr, nullptr, a.H, a.d, s,
                                     false);
                const size_t r = ((size_t)t * n_swa + si++) * ring_elems;
                sw.k_cache = a.k_rings + r;
                sw.v_cache = a.v_rings + r;
                if (e == hipSuccess) e = launch_swa_decode(sw, s);
            }
            if (e == hipSuccess) e = launch_gemm_resid(o, a.W_o[i], M, a.D, Hd, a.h, xb, s);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace lt2
