"""The allocation-free looped decode entry point (lt2_looped_decode_step_noalloc,
the library's fixed device scratch array instead of a workspace) against the
workspace entry point lt2_looped_decode_step, through the C ABI: two calls in a
row, the second with fewer sequences (the scratch array keeps the first call's
contents), each bit-identical to the workspace call on the same inputs."""
import numpy as np
import pytest
import torch

from linear_attention_looped_amd import lt2, synth
from gpu_util import TOL_BF16, announce, host, rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gate", [False, True])
def test_noalloc_decode_matches_workspace_entry_point(gate):
    D, H, d, T = 256, 2, 128, 2
    for call, B in enumerate((40, 17)):
        announce(f"noalloc looped decode gate={gate} call={call} B={B}")
        shape = synth.LoopShape(B, 1, D, H, d, T)
        w = synth.loop_weights(shape, seed=11, gate=gate)
        w_in = torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16)
        w_o = torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)
        rng = np.random.default_rng(100 + call)
        s0 = torch.from_numpy((rng.standard_normal((T, B, H, d, d)) * 0.05).astype(np.float32)).to("cuda")
        h0 = torch.from_numpy(synth.loop_h0(shape, seed=12 + call)[:, 0]).to("cuda")
        h_ref, s_ref = h0.clone(), s0.clone()
        lt2.lt2_looped_decode_step(h_ref, w_in, w_o, s_ref, H, d, T, out_gate=gate)
        h_new, s_new = h0.clone(), s0.clone()
        lt2.lt2_looped_decode_step_noalloc(h_new, w_in, w_o, s_new, H, d, T, out_gate=gate)
        torch.cuda.synchronize()
        assert rel_err(host(h_new), host(h_ref)) <= TOL_BF16
        np.testing.assert_array_equal(host(h_new), host(h_ref))
        np.testing.assert_array_equal(host(s_new), host(s_ref))


def test_noalloc_rejects_sizes_beyond_its_scratch():
    D, H, d, T = 2048, 16, 128, 1
    B = 2048                                  # layout of about 48 MiB > 32 MiB
    desc = lt2.loop_desc(B, 1, D, H, d, T, 64, 1)
    assert lt2.lt2_looped_decode_workspace_size(desc) > lt2.LT2_NOALLOC_SCRATCH_BYTES
    h = torch.zeros((B, D), dtype=torch.float32, device="cuda")
    w_in = torch.zeros((4 * H * d + 2 * H, D), dtype=torch.bfloat16, device="cuda")
    w_o = torch.zeros((D, H * d), dtype=torch.bfloat16, device="cuda")
    states = torch.zeros((T, B, H, d, d), dtype=torch.float32, device="cuda")
    with pytest.raises(lt2.Lt2Error, match="LT2_ERR_WORKSPACE"):
        lt2.lt2_looped_decode_step_noalloc(h, w_in, w_o, states, H, d, T, out_gate=True)
    assert torch.count_nonzero(h).item() == 0
