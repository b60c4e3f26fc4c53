"""GPU parity of the gated-delta backward pass with the per-channel gate
(lt2_gdn_backward with alpha [B, L, H, d_k], the KDA form) against the fp64
oracle's token adjoint.

Every gradient (dq, dk, dv, d log alpha per channel, d beta, dS_0) is compared
on its own: max|delta|/max|ref| <= 1e-5 for fp32 inputs, <= 5e-3 for bf16
inputs.  Shapes span several 16-token checkpoint segments with ragged tails,
both head sizes, initial states and final-state cotangents, extreme and exactly
zero decays; the per-channel workload (B1 H32 L32768 d128 bf16) runs whole and
is checked on sampled heads.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_looped_amd import lt2, synth
from gpu_util import TOL_BF16, TOL_F32, announce, dev, host, rel_err

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")


def run_bwd(x, dO, shape, S0=None, dSL=None, dO_dtype=None):
    qdt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    q, k, v = dev(x["q"], qdt), dev(x["k"], qdt), dev(x["v"], qdt)
    a, b = dev(x["alpha"]), dev(x["beta"])
    g = lt2.lt2_gdn_backward(q, k, v, a, b, dev(dO, dO_dtype or qdt), state_in=None if S0 is None else dev(S0),
                             d_state_out=None if dSL is None else dev(dSL))
    torch.cuda.synchronize()
    out = {n: host(g[n]) for n in ("dq", "dk", "dv", "dlog_alpha", "dbeta")}
    out["dS0"] = host(g["d_state_in"])
    return out


def check(got, ref, tol):
    for n in NAMES:
        print(f"  {n}:", end="")
        assert rel_err(got[n], ref[n]) <= tol, n


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [1, 17, 64, 100])
def test_channel_backward_fp32(d, L):
    shape = synth.GDNShape(2, L, 2, d, d, "channel", 0.0, "f32")
    announce(f"bwd channel fp32 d={d} L={L}")
    x = synth.gdn_inputs(shape, seed=21)
    dO = synth.grad_out(shape, seed=21)
    rng = np.random.default_rng(100 + L)
    S0 = rng.standard_normal((2, 2, d, d)).astype(np.float32)
    dSL = rng.standard_normal((2, 2, d, d)).astype(np.float32)
    got = run_bwd(x, dO, shape, S0, dSL)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, S0, dSL)
    check(got, ref, TOL_F32)


@pytest.mark.parametrize("d", [64, 128])
def test_channel_backward_bf16(d):
    shape = synth.GDNShape(2, 333, 2, d, d, "channel", 2.0, "bf16")
    announce(f"bwd channel bf16 d={d}")
    x = synth.gdn_inputs(shape, seed=22)
    dO = synth.grad_out(shape, seed=22)
    got = run_bwd(x, dO, shape)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO)
    check(got, ref, TOL_BF16)


def test_channel_backward_mixed_dtypes():
    """bf16 q, k, v with an fp32 output cotangent and both state terms."""
    shape = synth.GDNShape(1, 150, 3, 128, 128, "channel", 0.0, "bf16")
    announce("bwd channel bf16 inputs, fp32 cotangent")
    x = synth.gdn_inputs(shape, seed=23)
    dO = np.random.default_rng(23).standard_normal((1, 150, 3, 128)).astype(np.float32)
    rng = np.random.default_rng(24)
    S0 = (rng.standard_normal((1, 3, 128, 128)) * 0.1).astype(np.float32)
    dSL = rng.standard_normal((1, 3, 128, 128)).astype(np.float32)
    got = run_bwd(x, dO, shape, S0, dSL, dO_dtype=torch.float32)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, S0, dSL)
    check(got, ref, TOL_BF16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_channel_backward_extreme_gates(dtype):
    """Per-channel decays near 0 (shift 6) and near 1 (shift -6), then a mix:
    half the channels exactly 0 (the state forgets them every token; their
    log-alpha gradient is 0) and the rest near 1, with some tokens at beta = 0."""
    for case in ("fast", "slow", "mixed"):
        shift = {"fast": 6.0, "slow": -6.0, "mixed": 0.0}[case]
        shape = synth.GDNShape(1, 70, 2, 64, 64, "channel", shift, dtype)
        announce(f"bwd channel extreme gates {dtype} {case}")
        x = synth.gdn_inputs(shape, seed=25)
        if case == "mixed":
            x["alpha"][..., ::2] = 0.0
            x["alpha"][..., 1::2] = np.float32(0.999)
            x["beta"][:, ::7] = 0.0
        dO = synth.grad_out(shape, seed=25)
        got = run_bwd(x, dO, shape)
        ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO)
        check(got, ref, TOL_F32 if dtype == "f32" else TOL_BF16)
        if case == "mixed":
            assert np.all(got["dlog_alpha"][..., ::2] == 0.0)


def test_channel_gate_with_equal_channels_matches_scalar_gate():
    """A per-channel gate whose d_k entries all equal the head's scalar gate is
    the scalar gate: the two GPU backward paths (token adjoint on the vector
    ALUs, chunk form on the matrix cores) agree, the channel gate's log-alpha
    gradient summed over channels giving the scalar one."""
    shape = synth.GDNShape(2, 200, 2, 128, 128, "head", 0.0, "f32")
    announce("bwd channel == scalar for equal channels")
    x = synth.gdn_inputs(shape, seed=26)
    dO = synth.grad_out(shape, seed=26)
    g_head = run_bwd(x, dO, shape)
    xc = dict(x, alpha=np.ascontiguousarray(np.repeat(x["alpha"][..., None], 128, axis=-1)))
    g_chan = run_bwd(xc, dO, synth.GDNShape(2, 200, 2, 128, 128, "channel", 0.0, "f32"))
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        assert rel_err(g_chan[n], g_head[n]) <= TOL_F32, n
    assert rel_err(g_chan["dlog_alpha"].sum(axis=-1), g_head["dlog_alpha"]) <= TOL_F32


def test_channel_backward_full_workload_sampled_heads():
    """B1 H32 L32768 d128 bf16 with the per-channel gate (the per-channel
    prefill workload): the GPU runs all heads; the oracle recomputes two heads
    from their own streams."""
    shape = synth.WORKLOADS["channel_B1_H32_L32768_d128_bf16"]["shape"]
    announce("bwd channel full workload")
    x = synth.gdn_inputs(shape, seed=0)
    dO = synth.grad_out(shape, seed=0)
    got = run_bwd(x, dO, shape)
    del x
    for h in (0, 31):
        u = synth.gdn_unit(shape, 0, 0, h)
        du = synth.grad_out_unit(shape, 0, 0, h)
        ref = oracle.backward(u["q"][None, :, None], u["k"][None, :, None], u["v"][None, :, None],
                              u["alpha"][None, :, None], u["beta"][None, :, None], du[None, :, None])
        sub = {n: got[n][0:1, :, h:h + 1] for n in NAMES[:5]}
        sub["dS0"] = got["dS0"][0:1, h:h + 1]
        check(sub, ref, TOL_BF16)
