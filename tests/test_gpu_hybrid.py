"""GPU parity of the looped hybrid block (lt2_hybrid_mixer) against the oracle.

The shared block is a stack of gated-delta and sliding-window layers, applied
T times; the oracle runs it in fp64 with the same bf16-valued weights and h_0.
Bar: max|delta|/max|ref| <= 5e-3 on h_T (bf16 GEMM inputs, fp32 residual).
Exact properties checked on the GPU: a block of one gated-delta layer is the
looped mixer bit for bit, and a change of one token's input reaches, after T
loops of a window-w layer, exactly the tokens j .. j + T (w - 1) (the pages'
receptive field of O(T w)), every other output staying bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_looped_amd import lt2, synth
from gpu_util import TOL_BF16, announce, host, rel_err

pytestmark = pytest.mark.gpu


def make_layers(shape, kinds, seed, gate=False):
    host_layers, dev_layers = [], []
    for i, kind in enumerate(kinds):
        w = synth.loop_weights(shape, seed, gate, kind=kind, layer=i)
        host_layers.append((kind, w["w_in"], w["w_o"]))
        dev_layers.append((kind, torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16),
                           torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)))
    return host_layers, dev_layers


def run_hybrid(h0, dev_layers, shape, window, gate=False, chunk=64):
    h = torch.from_numpy(np.ascontiguousarray(h0, np.float32)).to("cuda")
    out = lt2.lt2_hybrid_mixer(h, dev_layers, shape.H, shape.d, shape.T, window, chunk=chunk, out_gate=gate)
    torch.cuda.synchronize()
    return host(out)


# At most four layer applications per case (the benchmarked hybrid is T = 2 of a
# two-layer block).  Every application rounds its GEMM and mixer inputs to bf16;
# a window layer's unnormalised q, k give large logits and its update roughly
# doubles max|h|, so the error against the fp64 oracle grows with depth.  An fp64
# emulation of these rounding points puts the full-size block at 2.2e-3 after
# four applications and at 3.9e-3 .. 5.4e-3 (by seed) after eight, which the
# 5e-3 bar does not hold reliably.
@pytest.mark.parametrize("kinds,gate,w,T", [(("gdn", "swa"), False, 64, 2), (("swa", "gdn"), True, 100, 2),
                                            (("swa",), False, 37, 2), (("gdn", "swa", "swa"), False, 300, 1)])
def test_hybrid_matches_oracle(kinds, gate, w, T):
    shape = synth.LoopShape(2, 333, 256, 2, 128, T)
    announce(f"hybrid {kinds} gate={gate} w={w} T={T}")
    hl, dl = make_layers(shape, kinds, seed=4, gate=gate)
    h0 = synth.loop_h0(shape, seed=4)
    got = run_hybrid(h0, dl, shape, w, gate)
    ref = oracle.hybrid_mixer(h0, hl, shape.H, shape.d, shape.T, w, gate=gate)
    assert rel_err(got, ref) <= TOL_BF16
    assert rel_err(got - h0, ref - h0) <= TOL_BF16


def test_hybrid_d64():
    shape = synth.LoopShape(1, 200, 128, 2, 64, 2)
    announce("hybrid d=64")
    hl, dl = make_layers(shape, ("gdn", "swa"), seed=5)
    h0 = synth.loop_h0(shape, seed=5)
    got = run_hybrid(h0, dl, shape, 50)
    ref = oracle.hybrid_mixer(h0, hl, shape.H, shape.d, shape.T, 50)
    assert rel_err(got, ref) <= TOL_BF16
    assert rel_err(got - h0, ref - h0) <= TOL_BF16


def test_gdn_only_block_is_the_looped_mixer_bitwise():
    shape = synth.LoopShape(1, 300, 256, 2, 128, 2)
    announce("hybrid gdn-only vs looped mixer")
    _, dl = make_layers(shape, ("gdn",), seed=6)
    h0 = synth.loop_h0(shape, seed=6)
    a = run_hybrid(h0, dl, shape, 1)
    h = torch.from_numpy(h0).to("cuda")
    b = host(lt2.lt2_looped_mixer(h, dl[0][1], dl[0][2], shape.H, shape.d, shape.T))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T,w", [(1, 40), (3, 40)])
def test_window_block_receptive_field_is_exactly_T_w(T, w):
    shape = synth.LoopShape(1, 600, 256, 2, 128, T)
    announce(f"hybrid receptive field T={T} w={w}")
    _, dl = make_layers(shape, ("swa",), seed=7)
    h0 = synth.loop_h0(shape, seed=7)
    j = 150
    h1 = h0.copy()
    h1[0, j] += 1.0
    d = np.abs(run_hybrid(h1, dl, shape, w) - run_hybrid(h0, dl, shape, w)).max(axis=2)[0]
    t = np.arange(shape.L)
    inside = (t >= j) & (t <= j + T * (w - 1))
    assert np.all(d[~inside] == 0.0)
    if T == 1:
        assert np.all(d[inside] > 0.0)        # every token of the window sees token j
    else:
        # later loops carry the change past the first loop's window (the reach
        # grows with T); far out the change can sink below bf16 resolution of
        # the GEMM inputs, so not every token of the field need move
        assert np.any(d[j + w:j + T * (w - 1) + 1] > 0.0)


def test_hybrid_full_size_prefix():
    """B=2 L=8192 d_model=2048 H=16 d=128, block (gated delta, window 512) looped
    T=2 times (four layer applications), the benchmarked launch shape: every
    layer is causal, so the oracle's run on the first 384 tokens of sequence 0
    must match the GPU's full run there."""
    s3 = synth.WORKLOADS["looped_B2_L8192_D2048_T4"]["shape"]
    shape = synth.LoopShape(s3.B, s3.L, s3.d_model, s3.H, s3.d, 2)
    announce("hybrid full size")
    hl, dl = make_layers(shape, ("gdn", "swa"), seed=0)
    h0 = synth.loop_h0(shape, seed=0)
    got = run_hybrid(h0, dl, shape, 512)
    P = 384
    ref = oracle.hybrid_mixer(h0[0:1, :P], hl, shape.H, shape.d, shape.T, 512)
    assert rel_err(got[0:1, :P], ref) <= TOL_BF16
    assert rel_err(got[0:1, :P] - h0[0:1, :P], ref - h0[0:1, :P]) <= TOL_BF16


@pytest.mark.parametrize("kinds,window,gate", [(("gdn", "swa"), 8, False), (("swa", "gdn"), 5, True),
                                               (("swa",), 3, False), (("gdn", "swa"), 64, False)])
def test_hybrid_decode_chain_matches_mixer(kinds, window, gate):
    """Token-by-token looped hybrid decode from zero states and empty rings gives,
    for every token, the h of the oracle's hybrid block on the whole sequence
    (every layer is causal); rings wrap when L > w, stay partly filled when
    L < w.  Four layer applications at most (T 2), as for the prefill cases."""
    B, L, D, H, d, T = 2, 24, 256, 2, 64, 2
    shape = synth.LoopShape(B, L, D, H, d, T)
    announce(f"hybrid decode chain kinds={kinds} w={window} gate={gate}")
    host_layers, dev_layers = make_layers(shape, kinds, seed=6, gate=gate)
    h0 = synth.loop_h0(shape, seed=6)
    ref = oracle.hybrid_mixer(h0, host_layers, H, d, T, window, gate=gate)
    n_gdn = sum(k == "gdn" for k in kinds)
    n_swa = len(kinds) - n_gdn
    states = torch.zeros((T, max(n_gdn, 1), B, H, d, d), dtype=torch.float32, device="cuda")[:, :n_gdn]
    kr = torch.zeros((T, max(n_swa, 1), B, H, window, d), dtype=torch.bfloat16, device="cuda")[:, :n_swa]
    vr = torch.zeros_like(kr)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    got = np.empty_like(h0)
    for t in range(L):
        h = torch.from_numpy(np.ascontiguousarray(h0[:, t], np.float32)).to("cuda")
        lt2.lt2_hybrid_decode_step(h, dev_layers, states.contiguous() if n_gdn else None, kr if n_swa else None,
                                   vr if n_swa else None, pos, H, d, T, window, out_gate=gate)
        got[:, t] = host(h)
        pos += 1
    torch.cuda.synchronize()
    assert rel_err(got, ref) <= TOL_BF16
    assert rel_err(got - h0, ref - h0) <= TOL_BF16
