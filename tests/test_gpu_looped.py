"""GPU parity of the looped LT2-linear block (lt2_looped_mixer) against the oracle.

The oracle runs the block in fp64 with the same bf16-valued weights and h_0; the
GPU rounds its GEMM inputs (bf16(h), q, k, v, o) to bf16 and keeps the residual
stream in fp32.  Bar: max|delta|/max|ref| <= 5e-3 on h_T (bf16 inputs, fp32 state).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_looped_amd import lt2, synth
from gpu_util import TOL_BF16, announce, host, rel_err

pytestmark = pytest.mark.gpu


def run_looped(h0, w, shape, chunk=64, gate=False):
    h = torch.from_numpy(np.ascontiguousarray(h0, np.float32)).to("cuda")
    w_in = torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16)
    w_o = torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)
    out = lt2.lt2_looped_mixer(h, w_in, w_o, shape.H, shape.d, shape.T, chunk=chunk, out_gate=gate)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("B,L,D,H,d,T", [(2, 200, 256, 2, 128, 2), (1, 333, 128, 2, 64, 3), (2, 64, 256, 4, 64, 1)])
def test_looped_small(B, L, D, H, d, T):
    shape = synth.LoopShape(B, L, D, H, d, T)
    announce(f"looped B={B} L={L} D={D} H={H} d={d} T={T}")
    w = synth.loop_weights(shape, seed=1)
    h0 = synth.loop_h0(shape, seed=1)
    got = run_looped(h0, w, shape)
    ref = oracle.looped_mixer(h0, w["w_in"], w["w_o"], H, d, T)
    assert rel_err(got, ref) <= TOL_BF16
    # the mixer's own contribution h_T - h_0, relative to its own scale
    assert rel_err(got - h0, ref - h0) <= TOL_BF16


def test_looped_zero_loops_is_identity():
    shape = synth.LoopShape(1, 100, 128, 2, 64, 0)
    announce("looped T=0")
    w = synth.loop_weights(shape, seed=2)
    h0 = synth.loop_h0(shape, seed=2)
    np.testing.assert_array_equal(run_looped(h0, w, shape), h0)


def test_looped_chunk_invariance():
    shape = synth.LoopShape(1, 160, 256, 2, 128, 2)
    announce("looped chunk 16 vs 64")
    w = synth.loop_weights(shape, seed=3)
    h0 = synth.loop_h0(shape, seed=3)
    a = run_looped(h0, w, shape, chunk=64)
    b = run_looped(h0, w, shape, chunk=16)
    ref = oracle.looped_mixer(h0, w["w_in"], w["w_o"], 2, 128, 2)
    assert rel_err(a, ref) <= TOL_BF16
    assert rel_err(b, ref) <= TOL_BF16


def test_looped_full_size_whole_sequence():
    """B=2 L=8192 d_model=2048 H=16 d=128 T=4 (the benchmarked launch, whose scan
    runs in 16-column blocks): sequences are independent, so the oracle's run
    on all 8192 tokens of sequence 1 alone must match the GPU's full run there,
    on h_T and on the mixers' contribution h_T - h_0."""
    shape = synth.WORKLOADS["looped_B2_L8192_D2048_T4"]["shape"]
    announce("looped full size, whole sequence 1")
    w = synth.loop_weights(shape, seed=0)
    h0 = synth.loop_h0(shape, seed=0)
    got = run_looped(h0, w, shape)
    assert np.all(np.isfinite(got))
    ref = oracle.looped_mixer(h0[1:2], w["w_in"], w["w_o"], shape.H, shape.d, shape.T)
    assert rel_err(got[1:2], ref) <= TOL_BF16
    assert rel_err(got[1:2] - h0[1:2], ref - h0[1:2]) <= TOL_BF16


@pytest.mark.parametrize("B,L,D,H,d,T", [(2, 40, 256, 2, 128, 2), (3, 17, 128, 2, 64, 3),
                                          (130, 6, 128, 2, 64, 2)])
def test_looped_decode_chain_matches_mixer(B, L, D, H, d, T):
    """Token-by-token looped decode from zero states gives, for every token, the
    h of the oracle's looped block on the whole sequence (each loop's mixer is
    causal, so its state after token t is the prefill state after token t)."""
    shape = synth.LoopShape(B, L, D, H, d, T)
    announce(f"looped decode chain B={B} L={L} D={D} H={H} d={d} T={T}")
    w = synth.loop_weights(shape, seed=4)
    h0 = synth.loop_h0(shape, seed=4)
    ref = oracle.looped_mixer(h0, w["w_in"], w["w_o"], H, d, T)
    w_in = torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16)
    w_o = torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)
    states = torch.zeros((T, B, H, d, d), dtype=torch.float32, device="cuda")
    got = np.empty_like(h0)
    for t in range(L):
        h = torch.from_numpy(np.ascontiguousarray(h0[:, t], np.float32)).to("cuda")
        lt2.lt2_looped_decode_step(h, w_in, w_o, states, H, d, T)
        got[:, t] = host(h)
    torch.cuda.synchronize()
    assert rel_err(got, ref) <= TOL_BF16
    assert rel_err(got - h0, ref - h0) <= TOL_BF16


def test_looped_decode_chain_full_width_sampled():
    """The decode chain at its benchmarked width (256 sequences, d_model 2048,
    H16 d128, T4: projection M 256 x N 6176 x K 2048 on the small-M GEMM, 32
    K-tiles through its LDS stages): two tokens for all sequences; the oracle
    recomputes the first and the last sequence on their own."""
    B, L, D, H, d, T = 256, 2, 2048, 16, 128, 4
    shape = synth.LoopShape(B, L, D, H, d, T)
    announce("looped decode chain full width")
    w = synth.loop_weights(shape, seed=3)
    h0 = synth.loop_h0(shape, seed=3)
    w_in = torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16)
    w_o = torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)
    states = torch.zeros((T, B, H, d, d), dtype=torch.float32, device="cuda")
    got = np.empty_like(h0)
    for t in range(L):
        h = torch.from_numpy(np.ascontiguousarray(h0[:, t], np.float32)).to("cuda")
        lt2.lt2_looped_decode_step(h, w_in, w_o, states, H, d, T)
        got[:, t] = host(h)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        ref = oracle.looped_mixer(h0[b:b + 1], w["w_in"], w["w_o"], H, d, T)
        assert rel_err(got[b:b + 1], ref) <= TOL_BF16, b
        assert rel_err(got[b:b + 1] - h0[b:b + 1], ref - h0[b:b + 1]) <= TOL_BF16, b


def test_looped_decode_equals_mixer_on_gpu():
    """Decode chain vs the GPU looped block on the same sequence (both bf16
    GEMM inputs, fp32 state): agreement far inside the oracle bar."""
    shape = synth.LoopShape(2, 24, 256, 2, 128, 2)
    announce("looped decode vs GPU mixer")
    w = synth.loop_weights(shape, seed=5)
    h0 = synth.loop_h0(shape, seed=5)
    full = run_looped(h0, w, shape)
    w_in = torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16)
    w_o = torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)
    states = torch.zeros((2, 2, 2, 128, 128), dtype=torch.float32, device="cuda")
    for t in range(shape.L):
        h = torch.from_numpy(np.ascontiguousarray(h0[:, t], np.float32)).to("cuda")
        lt2.lt2_looped_decode_step(h, w_in, w_o, states, 2, 128, 2)
        assert rel_err(host(h), full[:, t]) <= TOL_BF16, t


@pytest.mark.parametrize("B,L,D,H,d,T", [(2, 200, 256, 2, 128, 2), (1, 150, 128, 2, 64, 3)])
def test_looped_output_gate(B, L, D, H, d, T):
    """Looped block with the sigmoid output gate inside the loop."""
    shape = synth.LoopShape(B, L, D, H, d, T)
    announce(f"gated looped B={B} L={L} D={D} H={H} d={d} T={T}")
    w = synth.loop_weights(shape, seed=6, gate=True)
    h0 = synth.loop_h0(shape, seed=6)
    got = run_looped(h0, w, shape, gate=True)
    ref = oracle.looped_mixer(h0, w["w_in"], w["w_o"], H, d, T, gate=True)
    assert rel_err(got, ref) <= TOL_BF16
    assert rel_err(got - h0, ref - h0) <= TOL_BF16



def test_looped_output_gate_two_tiles_per_workgroup():
    """Gated looped block with 4 x 16 (b, h) units at d = 128: enough units for
    the column-tile scan's two-tiles-per-workgroup form, whose gated instance
    the smaller gated cases (one tile per workgroup) do not reach; ragged L."""
    shape = synth.LoopShape(4, 100, 256, 16, 128, 1)
    announce("gated looped, two column tiles per scan workgroup")
    w = synth.loop_weights(shape, seed=8, gate=True)
    h0 = synth.loop_h0(shape, seed=8)
    got = run_looped(h0, w, shape, gate=True)
    ref = oracle.looped_mixer(h0, w["w_in"], w["w_o"], 16, 128, 1, gate=True)
    assert rel_err(got, ref) <= TOL_BF16
    assert rel_err(got - h0, ref - h0) <= TOL_BF16

@pytest.mark.parametrize("L,D,H,d,gate", [(4000, 1024, 4, 128, True), (4000, 1024, 4, 128, False),
                                           (3000, 1024, 8, 64, True)])
def test_looped_large_tiles_ragged_rows(L, D, H, d, gate):
    """Shapes with enough 256 x 256 tiles for the large GEMM kernel (the smaller
    cases above run the small-M one), with rows that fill neither its 256-row
    tiles nor the 64-row short tiles of the last columns (the 2H gate-transform
    columns past N's last multiple of 256); gated and ungated, d = 128 and 64."""
    shape = synth.LoopShape(1, L, D, H, d, 1)
    announce(f"looped large tiles L={L} D={D} H={H} d={d} gate={gate}")
    w = synth.loop_weights(shape, seed=11, gate=gate)
    h0 = synth.loop_h0(shape, seed=11)
    got = run_looped(h0, w, shape, gate=gate)
    ref = oracle.looped_mixer(h0, w["w_in"], w["w_o"], H, d, 1, gate=gate)
    assert rel_err(got, ref) <= TOL_BF16
    assert rel_err(got - h0, ref - h0) <= TOL_BF16


def test_gated_looped_decode_chain_matches_mixer():
    shape = synth.LoopShape(2, 20, 256, 2, 128, 2)
    announce("gated looped decode chain")
    w = synth.loop_weights(shape, seed=7, gate=True)
    h0 = synth.loop_h0(shape, seed=7)
    ref = oracle.looped_mixer(h0, w["w_in"], w["w_o"], 2, 128, 2, gate=True)
    w_in = torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16)
    w_o = torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)
    states = torch.zeros((2, 2, 2, 128, 128), dtype=torch.float32, device="cuda")
    got = np.empty_like(h0)
    for t in range(shape.L):
        h = torch.from_numpy(np.ascontiguousarray(h0[:, t], np.float32)).to("cuda")
        lt2.lt2_looped_decode_step(h, w_in, w_o, states, 2, 128, 2, out_gate=True)
        got[:, t] = host(h)
    assert rel_err(got, ref) <= TOL_BF16
    assert rel_err(got - h0, ref - h0) <= TOL_BF16


def test_weight_layout_is_d_out_by_d_in():
    """The C ABI takes weights stored [d_out, d_in] and applies x W^T: with a
    square W_o (d_model = H*d = 256) the GPU block matches the oracle with that
    layout and is far from the same weights read as [d_in, d_out] (x W)."""
    shape = synth.LoopShape(1, 96, 256, 2, 128, 1)
    announce("weight layout")
    w = synth.loop_weights(shape, seed=8)
    h0 = synth.loop_h0(shape, seed=8)
    got = run_looped(h0, w, shape)
    ref = oracle.looped_mixer(h0, w["w_in"], w["w_o"], 2, 128, 1)
    ref_t = oracle.looped_mixer(h0, w["w_in"], np.ascontiguousarray(w["w_o"].T), 2, 128, 1)
    assert rel_err(got - h0, ref - h0) <= TOL_BF16
    assert rel_err(got - h0, ref_t - h0) > 0.1
