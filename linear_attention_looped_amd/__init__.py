"""MI355X (gfx950) mixers of LT2 (Linear-Time Looped Transformers): the gated
delta rule and sliding-window attention.

The compute lives in liblt2.so (hand-written HIP, C ABI in include/lt2.h);
this package only builds it (``build``), binds it (``lt2``) and draws seeded
synthetic inputs (``synth``).
"""
from .lt2 import (Lt2Error, lt2_gdn_backward, lt2_gdn_backward_workspace_size,  # noqa: F401
                  lt2_gdn_decode_step, lt2_gdn_prefill, lt2_gdn_prefill_workspace_size,
                  lt2_hbm_copy, lt2_hybrid_mixer, lt2_hybrid_mixer_workspace_size, lt2_looped_decode_step, lt2_looped_decode_workspace_size, lt2_looped_mixer,
                  lt2_looped_mixer_workspace_size, lt2_swa_prefill, status_string)
