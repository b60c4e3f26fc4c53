/* Drives the host-side argument validation of every liblt2 entry point under
 * AddressSanitizer and UndefinedBehaviorSanitizer (the library's host code
 * built with both; its GPU code is unchanged).  Every call here is refused, or
 * has nothing to do, before anything is enqueued, so no GPU is needed.  Exit
 * status 0 when every status matches. */
#include <stdint.h>
#include <stdio.h>

#include "lt2.h"

static int fails = 0;
#define EXPECT(call, code)                                                                   \
    do {                                                                                     \
        const int got_ = (int)(call);                                                        \
        if (got_ != (code)) {                                                                \
            fprintf(stderr, "%s:%d: %s -> %d, expected %d\n", __FILE__, __LINE__, #call, got_, \
                    (int)(code));                                                            \
            ++fails;                                                                         \
        }                                                                                    \
    } while (0)

#define F ((void *)(uintptr_t)0x10000)          /* aligned, never dereferenced */
#define FM ((void *)(uintptr_t)0x10004)         /* misaligned */

static lt2_gdn_desc gd(int B, int L, int H, int d, int chunk, int qd, int od, int gate) {
    lt2_gdn_desc x = {B, L, H, d, d, chunk, qd, od, gate};
    return x;
}
static lt2_loop_desc ld(int B, int L, int D, int H, int d, int T, int chunk, int gate) {
    lt2_loop_desc x = {B, L, D, H, d, T, chunk, gate};
    return x;
}

int main(void) {
    /* status strings, including unknown codes */
    for (int c = -1; c < 10; ++c)
        if (!lt2_status_string(c)) ++fails;

    /* prefill: descriptors at and past every limit */
    const int dims[][8] = {
        {2, 100, 3, 128, 64, 1, 1, 0}, {-1, 100, 3, 128, 64, 1, 1, 0}, {2, -1, 3, 128, 64, 1, 1, 0},
        {2, 100, 0, 128, 64, 1, 1, 0}, {2, 100, 3, 96, 64, 1, 1, 0},  {2, 100, 3, 128, 48, 1, 1, 0},
        {2, 100, 3, 128, 64, 9, 1, 0}, {2, 100, 3, 128, 64, 1, 1, 7},  {65535, 100, 65535, 128, 64, 1, 1, 0},
        {1, 2147483647, 1, 128, 16, 1, 1, 0}, {1, 2147483647, 1, 64, 64, 0, 0, 1},
        {1024, 1048576, 1024, 128, 16, 1, 1, 1}, {2147483647, 1, 1, 64, 16, 0, 0, 0},
    };
    const int expect[] = {LT2_OK, LT2_ERR_SHAPE, LT2_ERR_SHAPE, LT2_ERR_SHAPE, LT2_ERR_UNSUPPORTED,
                          LT2_ERR_UNSUPPORTED, LT2_ERR_DTYPE, LT2_ERR_UNSUPPORTED, LT2_ERR_SHAPE, LT2_ERR_SHAPE,
                          LT2_ERR_SHAPE, LT2_ERR_SHAPE, LT2_ERR_SHAPE};
    for (unsigned i = 0; i < sizeof(expect) / sizeof(expect[0]); ++i) {
        lt2_gdn_desc d = gd(dims[i][0], dims[i][1], dims[i][2], dims[i][3], dims[i][4], dims[i][5], dims[i][6],
                            dims[i][7]);
        const size_t ws = lt2_gdn_prefill_workspace_size(&d);
        const size_t wb = lt2_gdn_backward_workspace_size(&d);
        if (expect[i] == LT2_OK) {
            if (ws == 0 || wb == 0) ++fails;
            /* valid descriptor, workspace one byte short: refused before launching */
            EXPECT(lt2_gdn_prefill(&d, F, F, F, F, F, NULL, F, NULL, F, ws - 1, NULL), LT2_ERR_WORKSPACE);
            EXPECT(lt2_gdn_prefill_prepare(&d, F, F, F, F, F, ws - 1, NULL), LT2_ERR_WORKSPACE);
            EXPECT(lt2_gdn_prefill_scan(&d, F, F, F, NULL, F, NULL, F, ws - 1, NULL), LT2_ERR_WORKSPACE);
            EXPECT(lt2_gdn_prefill(&d, F, FM, F, F, F, NULL, F, NULL, F, ws, NULL), LT2_ERR_ALIGN);
            EXPECT(lt2_gdn_prefill(&d, F, F, F, NULL, F, NULL, F, NULL, F, ws, NULL), LT2_ERR_NULL);
            EXPECT(lt2_gdn_backward(&d, F, F, F, F, F, NULL, F, NULL, F, F, F, F, F, NULL, F, wb - 1, NULL),
                   LT2_ERR_WORKSPACE);
            d.gate = LT2_GATE_CHANNEL;
            const size_t wbc = lt2_gdn_backward_workspace_size(&d);
            if (wbc == 0) ++fails;
            EXPECT(lt2_gdn_backward(&d, F, F, F, F, F, NULL, F, NULL, F, F, F, F, F, NULL, F, wbc - 1, NULL),
                   LT2_ERR_WORKSPACE);
        } else {
            if (ws != 0 || wb != 0) ++fails;
            EXPECT(lt2_gdn_prefill(&d, F, F, F, F, F, NULL, F, NULL, F, (size_t)1 << 50, NULL), expect[i]);
            EXPECT(lt2_gdn_backward(&d, F, F, F, F, F, NULL, F, NULL, F, F, F, F, F, NULL, F, (size_t)1 << 50,
                                    NULL),
                   expect[i]);
        }
    }
    EXPECT(lt2_gdn_prefill(NULL, F, F, F, F, F, NULL, F, NULL, F, 0, NULL), LT2_ERR_NULL);
    {   /* nothing to do: empty batch */
        lt2_gdn_desc d = gd(0, 100, 3, 64, 64, 1, 1, 0);
        EXPECT(lt2_gdn_prefill(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), LT2_OK);
        EXPECT(lt2_gdn_backward(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                NULL, NULL, 0, NULL),
               LT2_OK);
    }
    /* decode */
    {
        lt2_gdn_desc d = gd(4, 2, 2, 64, 64, 1, 1, 0);
        EXPECT(lt2_gdn_decode_step(&d, F, F, F, F, F, F, F, NULL), LT2_ERR_SHAPE);
        d.L = 1;
        EXPECT(lt2_gdn_decode_step(&d, F, F, F, F, F, NULL, F, NULL), LT2_ERR_NULL);
        EXPECT(lt2_gdn_decode_step(&d, F, F, F, F, F, F, FM, NULL), LT2_ERR_ALIGN);
        d.B = 16384; d.H = 1024;
        EXPECT(lt2_gdn_decode_step(&d, F, F, F, F, F, F, F, NULL), LT2_ERR_SHAPE);
        d.B = 0;
        EXPECT(lt2_gdn_decode_step(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), LT2_OK);
    }
    /* looped block, looped decode (with and without a workspace), hybrid */
    {
        lt2_loop_desc d = ld(2, 100, 256, 2, 128, 2, 64, 0);
        const size_t w = lt2_looped_mixer_workspace_size(&d);
        if (w == 0) ++fails;
        EXPECT(lt2_looped_mixer(&d, F, F, F, F, F, w - 1, NULL), LT2_ERR_WORKSPACE);
        EXPECT(lt2_looped_mixer(&d, F, F, F, NULL, F, w, NULL), LT2_ERR_NULL);
        lt2_loop_desc bad = ld(2, 100, 192, 2, 128, 2, 64, 0);
        EXPECT(lt2_looped_mixer(&bad, F, F, F, F, F, w, NULL), LT2_ERR_UNSUPPORTED);
        if (lt2_looped_mixer_workspace_size(&bad) != 0) ++fails;
        lt2_loop_desc big = ld(4096, 524288, 256, 2, 128, 2, 16, 0);
        EXPECT(lt2_looped_mixer(&big, F, F, F, F, F, (size_t)1 << 60, NULL), LT2_ERR_SHAPE);
        lt2_loop_desc dd = ld(256, 1, 2048, 16, 128, 4, 64, 1);
        const size_t wd = lt2_looped_decode_workspace_size(&dd);
        if (wd == 0 || wd > LT2_NOALLOC_SCRATCH_BYTES) ++fails;
        EXPECT(lt2_looped_decode_step(&dd, F, F, F, F, F, wd - 1, NULL), LT2_ERR_WORKSPACE);
        lt2_loop_desc dbig = ld(2048, 1, 2048, 16, 128, 4, 64, 1);
        EXPECT(lt2_looped_decode_step_noalloc(&dbig, F, F, F, F, NULL), LT2_ERR_WORKSPACE);
        EXPECT(lt2_looped_decode_step_noalloc(&dd, F, F, F, NULL, NULL), LT2_ERR_NULL);
        dd.L = 2;
        EXPECT(lt2_looped_decode_step_noalloc(&dd, F, F, F, F, NULL), LT2_ERR_SHAPE);
        lt2_hybrid_desc hd = {1, 300, 256, 2, 128, 2, 64, 0, 64, 2, {LT2_MIXER_GDN, LT2_MIXER_SWA}};
        const void *wi[2] = {F, F}, *wo[2] = {F, F};
        const size_t wh = lt2_hybrid_mixer_workspace_size(&hd);
        EXPECT(lt2_hybrid_mixer(&hd, F, F, wi, wo, F, wh - 1, NULL), LT2_ERR_WORKSPACE);
        hd.n_layers = 9;
        EXPECT(lt2_hybrid_mixer(&hd, F, F, wi, wo, F, wh, NULL), LT2_ERR_SHAPE);
        hd.n_layers = 2; hd.kinds[1] = 5;
        EXPECT(lt2_hybrid_mixer(&hd, F, F, wi, wo, F, wh, NULL), LT2_ERR_UNSUPPORTED);
    }
    /* window attention and the bandwidth probes */
    {
        lt2_swa_desc s = {2, 300, 3, 128, 0, 1, 1};
        EXPECT(lt2_swa_prefill(&s, F, F, F, F, NULL), LT2_ERR_SHAPE);
        s.window = 64; s.L = 1 << 20; s.H = 16;
        EXPECT(lt2_swa_prefill(&s, F, F, F, F, NULL), LT2_ERR_SHAPE);
        s.L = 300; s.H = 3; s.qkv_dtype = 0;
        EXPECT(lt2_swa_prefill(&s, F, F, F, F, NULL), LT2_ERR_UNSUPPORTED);
        /* decode step: one token (L = 1) only; refused calls launch nothing */
        lt2_swa_desc sd = {2, 2, 3, 128, 64, 1, 1};
        EXPECT(lt2_swa_decode_step(&sd, F, F, F, F, F, (const int32_t *)F, F, NULL), LT2_ERR_SHAPE);
        sd.L = 1;
        sd.window = 0;
        EXPECT(lt2_swa_decode_step(&sd, F, F, F, F, F, (const int32_t *)F, F, NULL), LT2_ERR_SHAPE);
        sd.window = 64;
        EXPECT(lt2_swa_decode_step(&sd, F, F, F, NULL, F, (const int32_t *)F, F, NULL), LT2_ERR_NULL);
        sd.B = 0;
        EXPECT(lt2_swa_decode_step(&sd, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), LT2_OK);
        EXPECT(lt2_hbm_copy(F, F, 17, NULL), LT2_ERR_SHAPE);
        EXPECT(lt2_hbm_probe(F, F, 32, 7, 0, 4, NULL), LT2_ERR_UNSUPPORTED);
        EXPECT(lt2_hbm_probe(F, F, 32, 0, -5, 4, NULL), LT2_ERR_SHAPE);
        EXPECT(lt2_hbm_probe(F, NULL, 32, 1, 0, 4, NULL), LT2_ERR_NULL);
    }
    printf(fails ? "abi driver: %d FAILED\n" : "abi driver: ok\n", fails);
    return fails != 0;
}
