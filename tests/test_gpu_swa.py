"""GPU parity of the sliding-window attention kernel against the fp64 oracle.

Every case calls liblt2.so through its C ABI (the ctypes binding) on seeded
bf16 inputs and compares with ``oracle.swa``: max|delta|/max|ref| <= 5e-3 (the
bar of the bf16 workloads).  Shapes cover several 128-query workgroups and
64-key tiles, ragged tails, windows from 1 to beyond L, both head sizes and
both output types; the full workload (B2 L8192 H16 d128, window 512) is
checked on sampled query rows, each computed by the oracle on its own window.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_looped_amd import lt2, synth
from gpu_util import TOL_BF16, TOL_F32, announce, dev, host, rel_err

pytestmark = pytest.mark.gpu


def run_swa(x, window, out_dtype=torch.bfloat16):
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    o = lt2.lt2_swa_prefill(q, k, v, window, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,w", [(1, 1), (5, 3), (127, 16), (129, 64), (300, 100), (300, 1), (700, 128),
                                 (450, 257), (200, 1000)])
def test_swa_matches_oracle(d, L, w):
    shape = synth.SWAShape(2, L, 3, d, w)
    announce(f"swa d={d} L={L} w={w}")
    x = synth.swa_inputs(shape, seed=3)
    ref = oracle.swa(x["q"], x["k"], x["v"], w)
    assert rel_err(run_swa(x, w), ref) <= TOL_BF16
    assert rel_err(run_swa(x, w, torch.float32), ref) <= TOL_BF16


def test_swa_window_one_returns_values():
    """A window of one key: out = v up to the rounding of the scaled score that
    the kernel subtracts inside its exponent (relative 1e-6), for every element."""
    shape = synth.SWAShape(1, 333, 2, 128, 1)
    announce("swa w=1")
    x = synth.swa_inputs(shape, seed=4)
    np.testing.assert_allclose(run_swa(x, 1, torch.float32), x["v"].astype(np.float64), rtol=1e-6, atol=0)


def test_swa_peaked_scores():
    """Scores spread over tens of units: the running maximum changes inside and
    across tiles and the softmax is far from uniform."""
    shape = synth.SWAShape(1, 640, 2, 128, 300)
    announce("swa peaked scores")
    x = synth.swa_inputs(shape, seed=5)
    x["q"] = synth.bf16_round(x["q"] * 6.0)
    ref = oracle.swa(x["q"], x["k"], x["v"], 300)
    assert rel_err(run_swa(x, 300, torch.float32), ref) <= TOL_BF16


def test_swa_full_workload_sampled_rows():
    """B2 L8192 H16 d128, window 512, bf16 out, in the benchmark's launch
    configuration; query rows at tile, workgroup and window edges are checked
    against the oracle run on each row's own window."""
    shape = synth.SWA_WORKLOAD
    w = shape.window
    announce(f"swa full workload {shape}")
    x = synth.swa_inputs(shape, seed=0)
    o = run_swa(x, w)
    rows = [0, 1, 63, 64, 127, 128, 255, 510, 511, 512, 513, 1000, 4095, 4096, 8000, 8190, 8191]
    for b in range(shape.B):
        got, ref = [], []
        for t in rows:
            lo = max(0, t - w + 1)
            r = oracle.swa(x["q"][b:b + 1, lo:t + 1], x["k"][b:b + 1, lo:t + 1], x["v"][b:b + 1, lo:t + 1], w)
            ref.append(r[0, -1])
            got.append(o[b, t])
        assert rel_err(np.stack(got), np.stack(ref)) <= TOL_BF16


def test_swa_value_reaches_exactly_its_window_on_gpu():
    """Changing v_j changes exactly the outputs t = j .. j + w - 1; every other
    output is bit-identical (each output reads only its own window)."""
    shape = synth.SWAShape(1, 1024, 2, 128, 200)
    announce("swa value reach")
    x = synth.swa_inputs(shape, seed=6)
    o1 = run_swa(x, 200, torch.float32)
    j = 300
    x["v"] = x["v"].copy()
    x["v"][0, j] += 1.0
    o2 = run_swa(x, 200, torch.float32)
    diff = np.abs(o2 - o1).max(axis=(2, 3))[0]
    t = np.arange(1024)
    inside = (t >= j) & (t <= j + 199)
    assert np.all(diff[~inside] == 0.0)
    assert np.all(diff[inside] > 0.0)


# ---- decode form: one token per sequence against rings of the last w keys/values ----

def ring_history(g, B, H, w, d, pos):
    """Rings holding a random bf16 history of pos[b] tokens (token t at slot t % w)."""
    kc = np.zeros((B, H, w, d), np.float32)
    vc = np.zeros((B, H, w, d), np.float32)
    for b in range(B):
        for t in range(max(0, pos[b] - w), pos[b]):
            kc[b, :, t % w] = synth.bf16_round(g.standard_normal((H, d)).astype(np.float32) / np.sqrt(d))
            vc[b, :, t % w] = synth.bf16_round(g.standard_normal((H, d)).astype(np.float32))
    return kc, vc


@pytest.mark.parametrize("d,L,w", [(64, 40, 1), (128, 70, 16), (64, 70, 64), (128, 50, 100), (128, 130, 37)])
def test_swa_decode_chain_matches_oracle(d, L, w):
    """Token-by-token decode from empty rings equals the window attention of the
    whole sequence at every token (rings wrapping when L > w, partly filled
    when L < w); fp32 outputs at the fp32 bar (the inputs are bf16-valued, the
    arithmetic fp32), bf16 outputs at the bf16 bar."""
    B, H = 2, 3
    announce(f"swa decode chain d={d} L={L} w={w}")
    x = synth.swa_inputs(synth.SWAShape(B, L, H, d, w), seed=11)
    ref = oracle.swa(x["q"], x["k"], x["v"], w)
    for out_dtype, tol in ((torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)):
        kc = torch.zeros((B, H, w, d), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        pos = torch.zeros(B, dtype=torch.int32, device="cuda")
        q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
        outs = []
        for t in range(L):
            outs.append(lt2.lt2_swa_decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                                                kc, vc, pos, w, out_dtype=out_dtype))
            pos += 1
        torch.cuda.synchronize()
        got = np.stack([host(o) for o in outs], axis=1)
        assert rel_err(got, ref) <= tol, out_dtype


def test_swa_decode_ragged_positions():
    """Sequences at different positions (empty ring, partly filled, full, long
    past wrap-around) in one call: each output against the oracle's decode step,
    and the new key and value land in slot pos % w of each ring (bit-exact)."""
    g = np.random.default_rng(12)
    B, H, w, d = 4, 2, 37, 128
    pos = np.array([0, 5, 36, 200])
    announce(f"swa decode ragged positions {pos.tolist()} w={w}")
    kc, vc = ring_history(g, B, H, w, d, pos)
    q, k, v = (synth.bf16_round(g.standard_normal((B, H, d)).astype(np.float32)) for _ in range(3))
    kc_ref, vc_ref = kc.astype(np.float64), vc.astype(np.float64)
    ref = oracle.swa_decode_step(q, k, v, kc_ref, vc_ref, pos, w)
    tk, tv = dev(kc, torch.bfloat16), dev(vc, torch.bfloat16)
    out = lt2.lt2_swa_decode_step(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), tk, tv,
                                  torch.from_numpy(pos.astype(np.int32)).to("cuda"), w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_err(host(out), ref) <= TOL_F32
    np.testing.assert_array_equal(host(tk), kc_ref)
    np.testing.assert_array_equal(host(tv), vc_ref)


def test_swa_decode_full_size_rings():
    """A decode step of 16 sequences x 16 heads, d 128, window 512 on full rings
    (position 4095) against the oracle's decode step, bf16 output."""
    g = np.random.default_rng(13)
    B, H, w, d = 16, 16, 512, 128
    announce("swa decode full rings B16 H16 w512")
    kc = synth.bf16_round(g.standard_normal((B, H, w, d)).astype(np.float32) / np.sqrt(d))
    vc = synth.bf16_round(g.standard_normal((B, H, w, d)).astype(np.float32))
    q, k, v = (synth.bf16_round(g.standard_normal((B, H, d)).astype(np.float32)) for _ in range(3))
    pos = np.full(B, 4095)
    ref = oracle.swa_decode_step(q, k, v, kc.astype(np.float64), vc.astype(np.float64), pos, w)
    out = lt2.lt2_swa_decode_step(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16),
                                  dev(kc, torch.bfloat16), dev(vc, torch.bfloat16),
                                  torch.from_numpy(pos.astype(np.int32)).to("cuda"), w)
    torch.cuda.synchronize()
    assert rel_err(host(out), ref) <= TOL_BF16
