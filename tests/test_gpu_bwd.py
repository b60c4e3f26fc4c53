"""GPU parity of the gated-delta backward pass (lt2_gdn_backward, scalar gate)
against the fp64 oracle's token adjoint.

Every gradient (dq, dk, dv, d log alpha, d beta, dS_0) is compared on its own:
max|delta|/max|ref| <= 1e-5 for fp32 inputs, <= 5e-3 for bf16 inputs (the
bars of the forward workloads; the backward computes in fp32 from exactly
widened inputs).  Shapes span several 64-token chunks with ragged tails, both
head sizes, initial states and final-state cotangents; the full headline
workload (B4 H16 L4096 d128 bf16) is checked on sampled (b, h) units.
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
@pytest.mark.parametrize("L", [1, 37, 64, 65, 200])
def test_backward_fp32(d, L):
    shape = synth.GDNShape(2, L, 2, d, d, "head", 0.0, "f32")
    announce(f"bwd fp32 d={d} L={L}")
    x = synth.gdn_inputs(shape, seed=11)
    dO = synth.grad_out(shape, seed=11)
    rng = np.random.default_rng(L)
    S0 = rng.standard_normal((2, 2, d, d)).astype(np.float32)
    dSL = rng.standard_normal((2, 2, d, d)).astype(np.float32)
    got = run_bwd(x, dO, shape, S0, dSL)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, S0, dSL)
    check(got, ref, TOL_F32)


def test_backward_fp32_no_state():
    """S_0 = 0 and no final-state cotangent (the training case)."""
    shape = synth.GDNShape(1, 300, 3, 128, 128, "head", 2.0, "f32")
    announce("bwd fp32 no state")
    x = synth.gdn_inputs(shape, seed=12)
    dO = synth.grad_out(shape, seed=12)
    got = run_bwd(x, dO, shape)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO)
    check(got, ref, TOL_F32)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_bf16(d):
    shape = synth.GDNShape(2, 333, 2, d, d, "head", 2.0, "bf16")
    announce(f"bwd bf16 d={d}")
    x = synth.gdn_inputs(shape, seed=13)
    dO = synth.grad_out(shape, seed=13)
    got = run_bwd(x, dO, shape)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO)
    check(got, ref, TOL_BF16)


def test_backward_mixed_dtypes():
    """bf16 q, k, v with an fp32 output cotangent (bf16 matrix cores, dO split
    into hi + lo), and fp32 q, k, v with a bf16 cotangent (fp32 matrix cores)."""
    shape = synth.GDNShape(1, 150, 2, 128, 128, "head", 2.0, "bf16")
    announce("bwd bf16 inputs, fp32 dO")
    x = synth.gdn_inputs(shape, seed=15)
    dO = synth.grad_out(shape, seed=15)
    dO32 = np.random.default_rng(15).standard_normal(dO.shape).astype(np.float32)   # not bf16-valued
    got = run_bwd(x, dO32, shape, dO_dtype=torch.float32)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO32)
    check(got, ref, TOL_BF16)
    shape32 = synth.GDNShape(1, 150, 2, 64, 64, "head", 2.0, "f32")
    announce("bwd fp32 inputs, bf16 dO")
    x = synth.gdn_inputs(shape32, seed=16)
    dO = torch.from_numpy(synth.grad_out(shape32, seed=16)).to(torch.bfloat16).double().numpy()   # bf16-valued
    got = run_bwd(x, dO, shape32, dO_dtype=torch.bfloat16)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO)
    check(got, ref, TOL_F32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_extreme_gates(dtype):
    """alpha near 0 (shift 6: the state forgets every token) and near 1, beta in
    (0, 1): chunk-relative decays span hundreds of octaves inside a chunk (bf16:
    the split-operand matrix-core path over the same range)."""
    for shift in (6.0, -6.0):
        shape = synth.GDNShape(1, 130, 2, 64, 64, "head", shift, dtype)
        announce(f"bwd extreme gates {dtype} shift={shift}")
        x = synth.gdn_inputs(shape, seed=14)
        dO = synth.grad_out(shape, seed=14)
        got = run_bwd(x, dO, shape)
        ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO)
        check(got, ref, TOL_F32 if dtype == "f32" else TOL_BF16)


def test_backward_full_workload_sampled_units():
    """B4 H16 L4096 d128 bf16 (the headline prefill workload): the GPU runs the
    whole batch; the oracle recomputes two (b, h) units from their own streams."""
    shape = synth.WORKLOADS["prefill_B4_H16_L4096_d128_bf16"]["shape"]
    announce("bwd full workload")
    x = synth.gdn_inputs(shape, seed=0)
    dO = synth.grad_out(shape, seed=0)
    got = run_bwd(x, dO, shape)
    for b, h in ((0, 0), (3, 15)):
        u = synth.gdn_unit(shape, 0, b, h)
        du = synth.grad_out_unit(shape, 0, b, h)
        ref = oracle.backward(u["q"][None, :, None], u["k"][None, :, None], u["v"][None, :, None],
                              u["alpha"][None, :, None], u["beta"][None, :, None], du[None, :, None])
        sub = {n: got[n][b:b + 1, :, h:h + 1] for n in NAMES[:5]}
        sub["dS0"] = got["dS0"][b:b + 1, h:h + 1]
        check(sub, ref, TOL_BF16)
