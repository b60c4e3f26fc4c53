"""GPU parity of the gated-delta prefill and decode step against the fp64 oracle.

Every case calls liblt2.so through its C ABI (the ctypes binding) and compares
with oracle/ on the same seeded inputs: max|delta|/max|ref| <= 1e-5 for fp32
inputs and <= 5e-3 for bf16 inputs with fp32 state.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_looped_amd import lt2, synth
from gpu_util import TOL_BF16, TOL_F32, announce, dev, host, rel_err

pytestmark = pytest.mark.gpu


def run_prefill(x, shape, chunk, out_dtype=None, S0=None):
    qdt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    q, k, v = dev(x["q"], qdt), dev(x["k"], qdt), dev(x["v"], qdt)
    a, b = dev(x["alpha"]), dev(x["beta"])
    s0 = None if S0 is None else dev(S0)
    o, S = lt2.lt2_gdn_prefill(q, k, v, a, b, state_in=s0, chunk=chunk, out_dtype=out_dtype or qdt)
    torch.cuda.synchronize()
    return host(o), host(S)


def oracle_prefill(x, S0=None):
    return oracle.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0)


@pytest.mark.parametrize("chunk", [64, 32, 16])
def test_tiny_gdn_fp32_chunks(chunk):
    """B=1 H=1 L=256 d=64 fp32, scalar gate, S0=0: every chunk size matches the oracle."""
    shape = synth.WORKLOADS["prefill_B1_L256_d64_f32"]["shape"]
    announce(f"tiny fp32 chunk={chunk}")
    x = synth.gdn_inputs(shape, seed=0)
    o, S = run_prefill(x, shape, chunk)
    o_ref, S_ref = oracle_prefill(x)
    assert rel_err(o, o_ref) <= TOL_F32
    assert rel_err(S, S_ref) <= TOL_F32


@pytest.mark.parametrize("L", [1, 15, 37, 64, 65, 200])
@pytest.mark.parametrize("chunk", [16, 64])
def test_ragged_lengths_with_initial_state_fp32(L, chunk):
    shape = synth.GDNShape(2, L, 3, 64, 64, "head", 0.0, "f32")
    announce(f"ragged fp32 L={L} chunk={chunk}")
    x = synth.gdn_inputs(shape, seed=1)
    S0 = np.random.default_rng(1).standard_normal((2, 3, 64, 64)).astype(np.float32)
    o, S = run_prefill(x, shape, chunk, S0=S0)
    o_ref, S_ref = oracle_prefill(x, S0)
    assert rel_err(o, o_ref) <= TOL_F32
    assert rel_err(S, S_ref) <= TOL_F32


def test_fp32_d128_prefill():
    """d=128 fp32 (the state-seeding prefill of the decode workload)."""
    shape = synth.GDNShape(2, 300, 2, 128, 128, "head", 0.0, "f32")
    announce("fp32 d128")
    x = synth.gdn_inputs(shape, seed=2)
    o, S = run_prefill(x, shape, 64)
    o_ref, S_ref = oracle_prefill(x)
    assert rel_err(o, o_ref) <= TOL_F32
    assert rel_err(S, S_ref) <= TOL_F32


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_bf16_prefill_small(out_dtype):
    """bf16 q/k/v, fp32 state, strong decay (shift 2), ragged L spanning several chunks."""
    shape = synth.GDNShape(2, 333, 3, 128, 128, "head", 2.0, "bf16")
    announce(f"bf16 small out={out_dtype}")
    x = synth.gdn_inputs(shape, seed=3)
    S0 = np.random.default_rng(3).standard_normal((2, 3, 128, 128)).astype(np.float32) * 0.1
    o, S = run_prefill(x, shape, 64, out_dtype=out_dtype, S0=S0)
    o_ref, S_ref = oracle_prefill(x, S0)
    assert rel_err(o, o_ref) <= TOL_BF16
    assert rel_err(S, S_ref) <= TOL_BF16


def test_bf16_wide_and_narrow_column_blocks():
    """d128, chunk 64, bf16: 64 (b, h) units run the scan in 32-column blocks
    (256 workgroups); fewer units (here the first two batch rows alone, 32
    units) run it in 16-column blocks so that twice the workgroups fill the
    GPU.  Ragged L, initial state; both against the oracle."""
    shape = synth.GDNShape(4, 333, 16, 128, 128, "head", 2.0, "bf16")
    announce("bf16 wide and narrow column blocks")
    x = synth.gdn_inputs(shape, seed=21)
    S0 = np.random.default_rng(21).standard_normal((4, 16, 128, 128)).astype(np.float32) * 0.1
    o_ref, S_ref = oracle_prefill(x, S0)
    o, S = run_prefill(x, shape, 64, out_dtype=torch.float32, S0=S0)
    assert rel_err(o, o_ref) <= TOL_BF16
    assert rel_err(S, S_ref) <= TOL_BF16
    x2 = {kk: vv[:2] for kk, vv in x.items()}
    o2, S2 = run_prefill(x2, synth.GDNShape(2, 333, 16, 128, 128, "head", 2.0, "bf16"), 64,
                         out_dtype=torch.float32, S0=S0[:2])
    assert rel_err(o2, o_ref[:2]) <= TOL_BF16
    assert rel_err(S2, S_ref[:2]) <= TOL_BF16


def test_bf16_slow_decay_long():
    """bf16 with slow decay (shift 0), where the state carries over many chunks."""
    shape = synth.GDNShape(1, 1024, 2, 128, 128, "head", 0.0, "bf16")
    announce("bf16 slow decay")
    x = synth.gdn_inputs(shape, seed=4)
    o, S = run_prefill(x, shape, 64)
    o_ref, S_ref = oracle_prefill(x)
    assert rel_err(o, o_ref) <= TOL_BF16
    assert rel_err(S, S_ref) <= TOL_BF16



@pytest.mark.parametrize("shift", [2.0, -6.0])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_column_scan_output_precision_bf16(shift, out_dtype):
    """d128, chunk 64, bf16 q/k/v, 64 (b, h) units: the column-tile scan with two
    tiles per workgroup, on fast (shift 2) and slow (shift -6, alpha near 1)
    decays over eight whole chunks and a ragged one.  For bf16 outputs that scan
    takes Q S with the state's hi half only (Q S reaches only the outputs): the
    outputs hold the bf16 bar and the final state, which never sees that
    product, stays at the level of the fp32-output launch (1e-4)."""
    shape = synth.GDNShape(4, 555, 16, 128, 128, "head", shift, "bf16")
    announce(f"column scan output precision shift={shift} out={out_dtype}")
    x = synth.gdn_inputs(shape, seed=9)
    o, S = run_prefill(x, shape, 64, out_dtype=out_dtype)
    o_ref, S_ref = oracle_prefill(x)
    assert rel_err(o, o_ref) <= TOL_BF16
    assert rel_err(S, S_ref) <= 1e-4


def test_column_prepare_uneven_chunk_shares_bf16():
    """d128, chunk 64, bf16: 3 x 16 units of 1500 tokens = 1152 chunks, more than
    the prepare's grid of four workgroups per CU, so some workgroups take two
    chunks (the second one's K rows and gates prefetched during the first) and
    the others one; the last chunk of every unit is ragged (1500 = 23 x 64 + 28)."""
    shape = synth.GDNShape(3, 1500, 16, 128, 128, "head", 1.0, "bf16")
    announce("column prepare uneven shares")
    x = synth.gdn_inputs(shape, seed=12)
    S0 = np.random.default_rng(12).standard_normal((3, 16, 128, 128)).astype(np.float32) * 0.1
    o, S = run_prefill(x, shape, 64, S0=S0)
    o_ref, S_ref = oracle_prefill(x, S0)
    assert rel_err(o, o_ref) <= TOL_BF16
    assert rel_err(S, S_ref) <= TOL_BF16

def test_state_passing_and_chunk_invariance_bf16():
    shape = synth.GDNShape(1, 512, 2, 128, 128, "head", 0.0, "bf16")
    announce("state passing bf16")
    x = synth.gdn_inputs(shape, seed=5)
    o_full, S_full = run_prefill(x, shape, 64, out_dtype=torch.float32)
    L1 = 200
    xa = {kk: vv[:, :L1] for kk, vv in x.items()}
    xb = {kk: vv[:, L1:] for kk, vv in x.items()}
    oa, Sa = run_prefill(xa, synth.GDNShape(1, L1, 2, 128, 128, "head", 0.0, "bf16"), 64, out_dtype=torch.float32)
    ob, Sb = run_prefill(xb, synth.GDNShape(1, 512 - L1, 2, 128, 128, "head", 0.0, "bf16"), 32,
                         out_dtype=torch.float32, S0=Sa.astype(np.float32))
    assert rel_err(np.concatenate([oa, ob], axis=1), o_full) <= TOL_BF16
    assert rel_err(Sb, S_full) <= TOL_BF16
    o16, _ = run_prefill(x, shape, 16, out_dtype=torch.float32)
    assert rel_err(o16, o_full) <= TOL_BF16


def test_gate_special_cases_fp32():
    """alpha=1,beta=0 keeps S0; alpha=0 keeps only the current write (closed forms via the oracle)."""
    shape = synth.GDNShape(1, 100, 2, 64, 64, "head", 0.0, "f32")
    x = synth.gdn_inputs(shape, seed=6)
    S0 = np.random.default_rng(6).standard_normal((1, 2, 64, 64)).astype(np.float32)
    for name, a, b in (("a1b0", 1.0, 0.0), ("a0", 0.0, None), ("a1b1", 1.0, 1.0)):
        announce(f"special {name}")
        y = dict(x)
        y["alpha"] = np.full_like(x["alpha"], a)
        if b is not None:
            y["beta"] = np.full_like(x["beta"], b)
        o, S = run_prefill(y, shape, 64, S0=S0)
        o_ref, S_ref = oracle_prefill(y, S0)
        assert rel_err(o, o_ref) <= TOL_F32, name
        assert rel_err(S, S_ref) <= TOL_F32, name


@pytest.mark.parametrize("shift", [6.0, -6.0])
@pytest.mark.parametrize("chunk", [16, 64])
def test_fast_and_slow_scalar_gates_fp32(shift, chunk):
    """alpha = exp(-softplus(N(0,1) + 6)) (about e^-6: the state forgets almost
    every token, cumulative log2 gates reach hundreds of octaves inside a chunk)
    and shift -6 (alpha close to 1), fp32 inputs, to the fp32 bar."""
    shape = synth.GDNShape(2, 300, 2, 128, 128, "head", shift, "f32")
    announce(f"scalar gate shift={shift} chunk={chunk}")
    x = synth.gdn_inputs(shape, seed=41)
    S0 = np.random.default_rng(41).standard_normal((2, 2, 128, 128)).astype(np.float32)
    o, S = run_prefill(x, shape, chunk, S0=S0)
    o_ref, S_ref = oracle_prefill(x, S0)
    assert rel_err(o, o_ref) <= TOL_F32
    assert rel_err(S, S_ref) <= TOL_F32


def test_empty_and_determinism():
    announce("empty + determinism")
    shape = synth.GDNShape(1, 0, 2, 64, 64, "head", 0.0, "f32")
    x = synth.gdn_inputs(shape, seed=7)
    S0 = np.random.default_rng(7).standard_normal((1, 2, 64, 64)).astype(np.float32)
    o, S = run_prefill(x, shape, 64, S0=S0)
    assert o.shape == (1, 0, 2, 64)
    np.testing.assert_array_equal(S, S0)
    shape = synth.GDNShape(2, 250, 2, 128, 128, "head", 2.0, "bf16")
    x = synth.gdn_inputs(shape, seed=8)
    o1, S1 = run_prefill(x, shape, 64)
    o2, S2 = run_prefill(x, shape, 64)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_prefill_full_size_bf16_sampled():
    """B=4 H=16 L=4096 d=128 bf16, chunk 64 (the benchmarked prefill launch):
    sampled (b, h) units against the oracle."""
    shape = synth.WORKLOADS["prefill_B4_H16_L4096_d128_bf16"]["shape"]
    announce("prefill full size bf16")
    x = synth.gdn_inputs(shape, seed=0)
    o, S = run_prefill(x, shape, 64)
    for b, h in [(0, 0), (1, 7), (3, 15)]:
        u = synth.gdn_unit(shape, 0, b, h)
        o_ref, S_ref = oracle.prefill(u["q"][None, :, None], u["k"][None, :, None], u["v"][None, :, None],
                                      u["alpha"][None, :, None], u["beta"][None, :, None])
        assert rel_err(o[b, :, h], o_ref[0, :, 0]) <= TOL_BF16, (b, h)
        assert rel_err(S[b, h], S_ref[0, 0]) <= TOL_BF16, (b, h)


# ---- decode ---------------------------------------------------------------------

def run_decode(q, k, v, a, b, S, dtype=torch.float32):
    st = dev(S)
    o = lt2.lt2_gdn_decode_step(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(a), dev(b), st,
                                out=torch.empty(v.shape, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    return host(o), host(st)


@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_step_fp32(channel, d):
    announce(f"decode fp32 d={d} channel={channel}")
    rng = np.random.default_rng(20 + d + channel)
    B, H = 3, 5
    q = rng.standard_normal((B, H, d)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, H, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, d))
    a = rng.uniform(0.0, 1.0, (B, H, d) if channel else (B, H))
    b = rng.uniform(0.0, 1.0, (B, H))
    S = rng.standard_normal((B, H, d, d))
    args = [x.astype(np.float32) for x in (q, k, v, a, b, S)]
    o, S1 = run_decode(*args)
    o_ref, S_ref = oracle.decode_step(*args)
    assert rel_err(o, o_ref) <= TOL_F32
    assert rel_err(S1, S_ref) <= TOL_F32


def test_decode_chain_equals_prefill_bf16_inputs():
    """L decode steps reproduce a prefill over the same L tokens."""
    announce("decode chain vs prefill")
    shape = synth.GDNShape(2, 40, 3, 128, 128, "head", 0.0, "bf16")
    x = synth.gdn_inputs(shape, seed=9)
    o_ref, S_ref = oracle_prefill(x)
    st = torch.zeros((2, 3, 128, 128), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(40):
        o = lt2.lt2_gdn_decode_step(dev(x["q"][:, t], torch.bfloat16), dev(x["k"][:, t], torch.bfloat16),
                                    dev(x["v"][:, t], torch.bfloat16), dev(x["alpha"][:, t]),
                                    dev(x["beta"][:, t]), st,
                                    out=torch.empty((2, 3, 128), dtype=torch.float32, device="cuda"))
        outs.append(host(o))
    torch.cuda.synchronize()
    assert rel_err(np.stack(outs, axis=1), o_ref) <= TOL_F32
    assert rel_err(host(st), S_ref) <= TOL_F32


def test_decode_full_size_sampled():
    """256 sequences x 16 heads x d=128 fp32, 4 loops x 6 tokens of fresh inputs
    (the benchmarked decode launch), sampled units against the oracle."""
    announce("decode full size")
    B, H, d, T, steps = 256, 16, 128, 4, 6
    x = synth.decode_inputs(seed=3, B=B, H=H, T=T, steps=steps, d=d)
    S0 = np.random.default_rng(3).standard_normal((T, B, H, d, d)).astype(np.float32) * 0.05
    st = dev(S0)
    outs = np.empty((steps, T, B, H, d))
    for s in range(steps):
        for t in range(T):
            o = lt2.lt2_gdn_decode_step(dev(x["q"][s, t]), dev(x["k"][s, t]), dev(x["v"][s, t]),
                                        dev(x["alpha"][s, t]), dev(x["beta"][s, t]), st[t])
            outs[s, t] = host(o)
    torch.cuda.synchronize()
    S_fin = host(st)
    for (b, h, t) in [(0, 0, 0), (17, 5, 1), (255, 15, 3)]:
        u = synth.decode_unit(3, b, h, t, steps, d)
        o_ref, S_ref = oracle.prefill(u["q"][None, :, None], u["k"][None, :, None], u["v"][None, :, None],
                                      u["alpha"][None, :, None], u["beta"][None, :, None],
                                      S0[t, b, h][None, None])
        assert rel_err(outs[:, t, b, h], o_ref[0, :, 0]) <= TOL_F32, (b, h, t)
        assert rel_err(S_fin[t, b, h], S_ref[0, 0]) <= TOL_F32, (b, h, t)


# ---- per-channel gate (KDA form) ------------------------------------------------

@pytest.mark.parametrize("chunk", [64, 32, 16])
@pytest.mark.parametrize("shift", [0.0, 2.0])
def test_channel_gate_fp32(chunk, shift):
    shape = synth.GDNShape(2, 200, 3, 64, 64, "channel", shift, "f32")
    announce(f"channel fp32 chunk={chunk} shift={shift}")
    x = synth.gdn_inputs(shape, seed=30)
    S0 = np.random.default_rng(30).standard_normal((2, 3, 64, 64)).astype(np.float32)
    o, S = run_prefill(x, shape, chunk, S0=S0)
    o_ref, S_ref = oracle_prefill(x, S0)
    assert rel_err(o, o_ref) <= TOL_F32
    assert rel_err(S, S_ref) <= TOL_F32


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_channel_gate_bf16(out_dtype):
    shape = synth.GDNShape(1, 333, 2, 128, 128, "channel", 2.0, "bf16")
    announce(f"channel bf16 out={out_dtype}")
    x = synth.gdn_inputs(shape, seed=31)
    o, S = run_prefill(x, shape, 64, out_dtype=out_dtype)
    o_ref, S_ref = oracle_prefill(x)
    assert rel_err(o, o_ref) <= TOL_BF16
    assert rel_err(S, S_ref) <= TOL_BF16


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chunk", [64, 32, 16])
def test_channel_gate_bf16_chunks(d, chunk):
    """bf16 per-channel path at every chunk size and head width, ragged length,
    nonzero initial state."""
    shape = synth.GDNShape(2, 200, 2, d, d, "channel", 2.0, "bf16")
    announce(f"channel bf16 d={d} chunk={chunk}")
    x = synth.gdn_inputs(shape, seed=35 + d + chunk)
    S0 = np.random.default_rng(35).standard_normal((2, 2, d, d)).astype(np.float32)
    o, S = run_prefill(x, shape, chunk, out_dtype=torch.float32, S0=S0)
    o_ref, S_ref = oracle_prefill(x, S0)
    assert rel_err(o, o_ref) <= TOL_BF16
    assert rel_err(S, S_ref) <= TOL_BF16


@pytest.mark.parametrize("case", ["zero", "some_channels_near_zero", "one"])
def test_channel_gate_extreme_decays_bf16(case):
    """bf16 inputs with the gate extremes of the fp32 case (a block whose gate span
    exceeds the matrix-core reference range is summed pair by pair)."""
    shape = synth.GDNShape(1, 150, 2, 128, 128, "channel", 0.0, "bf16")
    announce(f"channel bf16 extreme {case}")
    x = synth.gdn_inputs(shape, seed=36)
    a = x["alpha"].copy()
    if case == "zero":
        a[:] = 0.0
    elif case == "one":
        a[:] = 1.0
    else:
        a[..., ::7] = 1e-20
    x["alpha"] = a
    S0 = np.random.default_rng(36).standard_normal((1, 2, 128, 128)).astype(np.float32)
    o, S = run_prefill(x, shape, 64, out_dtype=torch.float32, S0=S0)
    o_ref, S_ref = oracle_prefill(x, S0)
    assert rel_err(o, o_ref) <= TOL_BF16
    assert rel_err(S, S_ref) <= TOL_BF16


def test_channel_gate_slow_decay_d128_fp32():
    shape = synth.GDNShape(1, 300, 2, 128, 128, "channel", 0.0, "f32")
    announce("channel fp32 d128 slow decay")
    x = synth.gdn_inputs(shape, seed=32)
    o, S = run_prefill(x, shape, 64)
    o_ref, S_ref = oracle_prefill(x)
    assert rel_err(o, o_ref) <= TOL_F32
    assert rel_err(S, S_ref) <= TOL_F32


@pytest.mark.parametrize("case", ["zero", "some_channels_near_zero", "one"])
def test_channel_gate_extreme_decays_fp32(case):
    """alpha = 0 everywhere, a few channels with alpha ~ 1e-20 (gate spans far past
    the matrix-core reference range inside a block), and alpha = 1."""
    shape = synth.GDNShape(1, 150, 2, 64, 64, "channel", 0.0, "f32")
    announce(f"channel extreme {case}")
    x = synth.gdn_inputs(shape, seed=33)
    a = x["alpha"].copy()
    if case == "zero":
        a[:] = 0.0
    elif case == "one":
        a[:] = 1.0
    else:
        a[..., ::7] = 1e-20
    x["alpha"] = a
    S0 = np.random.default_rng(33).standard_normal((1, 2, 64, 64)).astype(np.float32)
    o, S = run_prefill(x, shape, 64, S0=S0)
    o_ref, S_ref = oracle_prefill(x, S0)
    assert rel_err(o, o_ref) <= TOL_F32
    assert rel_err(S, S_ref) <= TOL_F32


def test_channel_state_passing_bf16():
    shape = synth.GDNShape(1, 256, 2, 128, 128, "channel", 2.0, "bf16")
    announce("channel state passing")
    x = synth.gdn_inputs(shape, seed=34)
    o_full, S_full = run_prefill(x, shape, 64, out_dtype=torch.float32)
    L1 = 100
    xa = {kk: vv[:, :L1] for kk, vv in x.items()}
    xb = {kk: vv[:, L1:] for kk, vv in x.items()}
    oa, Sa = run_prefill(xa, synth.GDNShape(1, L1, 2, 128, 128, "channel", 2.0, "bf16"), 64, out_dtype=torch.float32)
    ob, Sb = run_prefill(xb, synth.GDNShape(1, 256 - L1, 2, 128, 128, "channel", 2.0, "bf16"), 64,
                         out_dtype=torch.float32, S0=Sa.astype(np.float32))
    assert rel_err(np.concatenate([oa, ob], axis=1), o_full) <= TOL_BF16
    assert rel_err(Sb, S_full) <= TOL_BF16


def test_channel_full_size_bf16_sampled():
    """B=1 H=32 L=32768 d=128 bf16, per-channel gate (the benchmarked launch):
    sampled heads against the oracle."""
    shape = synth.WORKLOADS["channel_B1_H32_L32768_d128_bf16"]["shape"]
    announce("channel full size")
    x = synth.gdn_inputs(shape, seed=0)
    o, S = run_prefill(x, shape, 64)
    for h in (0, 31):
        u = synth.gdn_unit(shape, 0, 0, h)
        o_ref, S_ref = oracle.prefill(u["q"][None, :, None], u["k"][None, :, None], u["v"][None, :, None],
                                      u["alpha"][None, :, None], u["beta"][None, :, None])
        assert rel_err(o[0, :, h], o_ref[0, :, 0]) <= TOL_BF16, h
        assert rel_err(S[0, h], S_ref[0, 0]) <= TOL_BF16, h


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prepare_then_scan_equals_prefill(gate):
    """lt2_gdn_prefill_prepare followed by lt2_gdn_prefill_scan (which receives no
    alpha or beta) gives exactly what lt2_gdn_prefill gives."""
    import ctypes
    shape = synth.GDNShape(2, 150, 2, 128, 128, gate, 2.0, "bf16")
    announce(f"phases {gate}")
    x = synth.gdn_inputs(shape, seed=40)
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    a, b = dev(x["alpha"]), dev(x["beta"])
    o_ref, S_ref = lt2.lt2_gdn_prefill(q, k, v, a, b, chunk=64, out_dtype=torch.float32)
    desc = lt2.gdn_desc(2, 150, 2, 128, 128, 64, lt2.LT2_BF16, lt2.LT2_F32,
                        lt2.LT2_GATE_CHANNEL if gate == "channel" else lt2.LT2_GATE_HEAD)
    nbytes = lt2.lt2_gdn_prefill_workspace_size(desc)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(o_ref)
    S = torch.empty_like(S_ref)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L_ = lt2.lib()
    assert L_.lt2_gdn_prefill_prepare(ctypes.byref(desc), P(q), P(k), P(a), P(b), P(ws), nbytes, sp) == 0
    assert L_.lt2_gdn_prefill_scan(ctypes.byref(desc), P(q), P(k), P(v), None, P(o), P(S), P(ws), nbytes, sp) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o), host(o_ref))
    np.testing.assert_array_equal(host(S), host(S_ref))


@pytest.mark.parametrize("L", [333, 64, 1])
def test_column_scan_phases_bf16(L):
    """d128, chunk 64, bf16 in and out, 64 (b, h) units: the column-tile path,
    whose scan workgroups form each chunk's gated Q K^T themselves (the prepare
    phase writes only the inverse factor and the gate prefix).  lt2_gdn_prefill
    with the final state written in place over the initial one equals its two
    phases called apart (lt2_gdn_prefill_prepare, then lt2_gdn_prefill_scan) bit
    for bit, and the oracle within the bf16 bound.  Ragged, single-chunk and
    single-token lengths."""
    import ctypes
    B, H = 4, 16
    shape = synth.GDNShape(B, L, H, 128, 128, "head", 2.0, "bf16")
    announce(f"column scan phases L={L}")
    x = synth.gdn_inputs(shape, seed=23)
    S0 = np.random.default_rng(23).standard_normal((B, H, 128, 128)).astype(np.float32) * 0.1
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    a, b = dev(x["alpha"]), dev(x["beta"])
    st = dev(S0)
    o1, _ = lt2.lt2_gdn_prefill(q, k, v, a, b, state_in=st, state_out=st, chunk=64, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    desc = lt2.gdn_desc(B, L, H, 128, 128, 64, lt2.LT2_BF16, lt2.LT2_BF16, lt2.LT2_GATE_HEAD)
    nbytes = lt2.lt2_gdn_prefill_workspace_size(desc)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    S2 = torch.empty_like(st)
    s0 = dev(S0)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L_ = lt2.lib()
    assert L_.lt2_gdn_prefill_prepare(ctypes.byref(desc), P(q), P(k), P(a), P(b), P(ws), nbytes, sp) == 0
    assert L_.lt2_gdn_prefill_scan(ctypes.byref(desc), P(q), P(k), P(v), P(s0), P(o2), P(S2), P(ws), nbytes, sp) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o1), host(o2))
    np.testing.assert_array_equal(host(st), host(S2))
    o_ref, S_ref = oracle_prefill(x, S0)
    assert rel_err(host(o1), o_ref) <= TOL_BF16
    assert rel_err(host(st), S_ref) <= TOL_BF16


@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_state_in_place(gate, dtype):
    """state_out may be the state_in buffer (the header allows it): with a ragged
    L the in-place call gives, bit for bit, what separate buffers give, and both
    match the oracle."""
    shape = synth.GDNShape(2, 150, 2, 128, 128, gate, 0.0, dtype)
    announce(f"in-place state {gate} {dtype}")
    x = synth.gdn_inputs(shape, seed=41)
    S0 = np.random.default_rng(41).standard_normal((2, 2, 128, 128)).astype(np.float32) * 0.1
    qdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (dev(x[n], qdt) for n in ("q", "k", "v"))
    a, b = dev(x["alpha"]), dev(x["beta"])
    o1, S1 = lt2.lt2_gdn_prefill(q, k, v, a, b, state_in=dev(S0), chunk=64, out_dtype=torch.float32)
    st = dev(S0)
    o2, S2 = lt2.lt2_gdn_prefill(q, k, v, a, b, state_in=st, state_out=st, chunk=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert S2.data_ptr() == st.data_ptr()
    np.testing.assert_array_equal(host(o2), host(o1))
    np.testing.assert_array_equal(host(st), host(S1))
    o_ref, S_ref = oracle_prefill(x, S0)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert rel_err(host(o2), o_ref) <= tol
    assert rel_err(host(st), S_ref) <= tol


@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [16, 64])
def test_workspace_nan_canary(gate, dtype, chunk):
    """The scan reads only workspace bytes the prepare phase wrote: a workspace
    filled with NaN beforehand gives finite outputs bit-identical to a
    zero-filled one, on a ragged last chunk."""
    L = 150 if chunk == 64 else 71
    shape = synth.GDNShape(1, L, 3, 64, 64, gate, 0.0, dtype)
    announce(f"nan canary {gate} {dtype} chunk={chunk}")
    x = synth.gdn_inputs(shape, seed=42)
    qdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (dev(x[n], qdt) for n in ("q", "k", "v"))
    a, b = dev(x["alpha"]), dev(x["beta"])
    desc = lt2.gdn_desc(1, L, 3, 64, 64, chunk, lt2._dt(q), lt2.LT2_F32,
                        lt2.LT2_GATE_CHANNEL if gate == "channel" else lt2.LT2_GATE_HEAD)
    nbytes = lt2.lt2_gdn_prefill_workspace_size(desc)
    res = []
    for fill in (0x00, 0xFF):          # 0xFF bytes: NaN as fp32 and as bf16
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        o, S = lt2.lt2_gdn_prefill(q, k, v, a, b, chunk=chunk, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        res.append((host(o), host(S)))
    for arr in res[1]:
        assert np.all(np.isfinite(arr))
    np.testing.assert_array_equal(res[1][0], res[0][0])
    np.testing.assert_array_equal(res[1][1], res[0][1])
