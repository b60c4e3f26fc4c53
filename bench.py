#!/usr/bin/env python3
"""Benchmark of the LT2 gated-delta hot path on one MI355X; prints ONE JSON line.

Headline workload (the step that is timed K times): one chunked gated-delta
prefill, B=4 H=16 L=4096 d_k=d_v=128, bf16 q/k/v, fp32 state, chunk 64, T=1
(scalar gate exp(-softplus(N(0,1)+2))).  value = tokens/s per loop = B*L*T / t.
Inputs are seeded, synthetic and resident in HBM before timing; two input sets
alternate so that no step re-reads the previous step's data from cache.

roofline: the dominant kernel of the step (the scan), HIP events on its launch
stream, against the 8 TB/s HBM peak, with the path's algorithmic bytes
(q, k, v, alpha, beta read once, o written once, the final state: 1032 B per
head-token + 4 B per state element); its measured HBM traffic comes from the
committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs (profiles/traffic.json).

Also measured in the same run (reported under "extra"):
  * the per-kernel split of the prefill (prepare / scan) from HIP events;
  * HBM probes: streaming copy (grid-stride by element and by per-workgroup
    tile), read-only and write-only kernels over a sweep of grid sizes and
    unroll depths; the best copy is the measured ceiling;
  * decode: 256 sequences x 16 heads x d=128, fp32 state from a seeded 2048-token
    prefill, T=4 loops per token, 1024 tokens with fresh inputs; one
    lt2_gdn_decode_step launch per (token, loop); state GB/s against HBM peak and
    against the measured copy ceiling;
  * the looped block (T=4), with and without the output gate; the looped decode
    chain; the per-channel-gate prefill; window attention and its decode step
    (ring of the last 512 keys and values); the looped hybrid
    block (gated delta, window 512) at T=2 (four layer applications, the depth
    its parity tests cover) and its decode chain; the backward pass of the
    headline workload.
cpu_baseline: the fp64 oracle on the whole headline workload (16,384 tokens x
16 heads), passes repeated for at least 5 s, timed on the host cores (their
count and model recorded).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] ...
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

METRIC = "gated-delta tokens/s per loop (prefill) + decode state GB/s vs HBM peak"
ROOT = os.path.dirname(os.path.abspath(__file__))
# sources whose kernels the counter runs in profiles/traffic.json measured
KERNEL_SOURCES = {
    "prepare": ["linear_attention_looped_amd/csrc/prefill_head.hip", "linear_attention_looped_amd/csrc/common.h"],
    "scan": ["linear_attention_looped_amd/csrc/prefill_head.hip", "linear_attention_looped_amd/csrc/common.h"],
}
TRAFFIC_KEYS = {"prepare": "prep_col_kernel", "scan": "scan_head_col_kernel"}
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# fp32 FMA on the vector ALUs without packed-fp32 instructions: 256 CUs x 4 SIMDs
# x 16 lanes x 2 flop x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 78.6


def measured_traffic(kernel: str):
    """HBM bytes per launch of the headline kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE runs (profiles/traffic.json, calibrated on the copy
    probe), or None when the kernel's sources changed since they were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)["kernels"][TRAFFIC_KEYS[kernel]]
        h = hashlib.sha256()
        for src in KERNEL_SOURCES[kernel]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        return rec["bytes"] if h.hexdigest()[:16] == rec["src_sha256_16"] else None
    except (OSError, KeyError, ValueError):
        return None


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_flops_bytes(B, L, H, d, C, qkv_bytes=2, out_bytes=2):
    """Algorithmic flops and bytes per kernel of the chunked prefill (per launch),
    as the two kernels of the d = 128, C = 64 bf16 path split the work.

    prepare, per head-token: gated K K^T (strictly lower) C*d/2 MACs, the
      unit-lower inverse C^2/6 MACs; reads k, alpha, beta; writes the chunk's
      workspace (the lower Tm fragments as bf16 hi/lo pairs, 12 KiB, the fp64 gate
      prefix and the two decay vectors, 1 KiB: 13,312 bytes per 64-token chunk).
    scan, per head-token: K S, Q S and K^T U (3*d*d MACs), Tm R and P U (C*d MACs),
      the gated Q K^T (lower incl., C*d/2 MACs); reads q, k, v and the workspace;
      writes o; reads/writes the state once per unit.
    """
    ht = B * L * H
    prep_flops = 2.0 * ht * (C * d / 2.0 + C * C / 6.0)
    scan_flops = 2.0 * ht * (3.0 * d * d + C * d + C * d / 2.0)
    ws_per_ht = 13312.0 / C
    prep_bytes = ht * (d * qkv_bytes + 8 + ws_per_ht)
    scan_bytes = ht * (3 * d * qkv_bytes + ws_per_ht + d * out_bytes) + B * H * d * d * 4.0
    path_bytes = ht * (3 * d * qkv_bytes + 8 + d * out_bytes) + B * H * d * d * 4.0
    # the method's own flops per head-token of the chunk form: K K^T, Q K^T and
    # Tm (gamma K) (C d_k each), Tm V and P U (C d_v each), W S, (gamma Q) S and
    # K^T U (d_k d_v each), the inverse (C^2 / 6)
    path_flops = 2.0 * ht * (C * (3 * d + 2 * d) + 3 * d * d + C * C / 6.0)
    return dict(prepare=(prep_flops, prep_bytes), scan=(scan_flops, scan_bytes), path_bytes=path_bytes,
                path_flops=path_flops)


def bench_prefill(args, torch, lt2, synth):
    cfg = synth.WORKLOADS["prefill_B4_H16_L4096_d128_bf16"]
    shape, C = cfg["shape"], cfg["chunk"]
    B, L, H, d = shape.B, shape.L, shape.H, shape.dk
    log(f"prefill inputs B={B} L={L} H={H} d={d} (2 seeded sets)")
    sets = []
    for seed in (0, 1):
        x = synth.gdn_inputs(shape, seed=seed)
        sets.append(dict(q=torch.from_numpy(x["q"]).to("cuda").to(torch.bfloat16),
                         k=torch.from_numpy(x["k"]).to("cuda").to(torch.bfloat16),
                         v=torch.from_numpy(x["v"]).to("cuda").to(torch.bfloat16),
                         alpha=torch.from_numpy(x["alpha"]).to("cuda"),
                         beta=torch.from_numpy(x["beta"]).to("cuda")))
        del x
    out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    desc = lt2.gdn_desc(B, L, H, d, d, C, lt2.LT2_BF16, lt2.LT2_BF16, lt2.LT2_GATE_HEAD)
    ws_bytes = lt2.lt2_gdn_prefill_workspace_size(desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    L_ = lt2.lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    calls = []
    for s in sets:
        calls.append(((ctypes.byref(desc), P(s["q"]), P(s["k"]), P(s["alpha"]), P(s["beta"]), P(ws), ws_bytes, sp),
                      (ctypes.byref(desc), P(s["q"]), P(s["k"]), P(s["v"]), None, P(out), P(S), P(ws), ws_bytes, sp)))

    def step(i, ev=None):
        prep, scan = calls[i % 2]
        if ev is not None:
            ev[0].record(stream)
        rc = L_.lt2_gdn_prefill_prepare(*prep)
        if ev is not None:
            ev[1].record(stream)
        rc |= L_.lt2_gdn_prefill_scan(*scan)
        if ev is not None:
            ev[2].record(stream)
        if rc:
            raise RuntimeError(f"prefill failed rc={rc}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    event_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in evs]))
    fb = prefill_flops_bytes(B, L, H, d, C)
    log(f"prefill {ms_step:.3f} ms/step (events {event_ms:.3f}: prepare {prep_ms:.3f}, scan {scan_ms:.3f})")
    kernels = {}
    for name, ms in (("prepare", prep_ms), ("scan", scan_ms)):
        fl, by = fb[name]
        kernels[name] = dict(ms=ms, flops=fl, bytes=by, tflops=fl / ms / 1e9, gbs=by / ms / 1e6)
    return dict(B=B, L=L, H=H, d=d, C=C, ms_step=ms_step, event_ms=event_ms, kernels=kernels,
                path_bytes=fb["path_bytes"], path_flops=fb["path_flops"], ws_bytes=ws_bytes)


def bench_copy(torch, lt2, nbytes=2 << 30, reps=5):
    """HBM probes over a sweep of launch shapes (workgroups of 256 lanes x
    16-byte accesses in flight per lane): streaming copy (read + write) grid-
    stride by element and by contiguous per-workgroup tile, read only, write
    only, each on 2 GiB buffers; per mode the best median is the measured
    ceiling, reported with its shape."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {}
    for mode, name, moved in ((lt2.PROBE_COPY, "copy", 2 * nbytes), (lt2.PROBE_TILE_COPY, "tile_copy", 2 * nbytes),
                              (lt2.PROBE_READ, "read", nbytes), (lt2.PROBE_WRITE, "write", nbytes)):
        best = None
        for per_cu in (4, 8, 16, 32):
            for unroll in (2, 4, 8, 16):
                blocks = per_cu * cus
                for _ in range(2):
                    lt2.lt2_hbm_probe(b, a, mode, blocks, unroll)
                times = []
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    lt2.lt2_hbm_probe(b, a, mode, blocks, unroll)
                    e1.record()
                    e1.synchronize()
                    times.append(e0.elapsed_time(e1))
                ms = float(np.median(times))
                gbs = moved / ms / 1e6
                if best is None or gbs > best["gbs"]:
                    best = dict(gbs=gbs, ms=ms, bytes_moved=moved, blocks=blocks, unroll=unroll)
        res[name] = best
        log(f"probe {name}: best {best['gbs']:.0f} GB/s ({best['blocks']} workgroups, unroll {best['unroll']})")
    del a, b
    torch.cuda.empty_cache()
    # the measured copy ceiling: the better of the two copy patterns
    res["gbs"] = max(res["copy"]["gbs"], res["tile_copy"]["gbs"])
    return res


def bench_decode(args, torch, lt2, synth):
    cfg = synth.WORKLOADS["decode_B256_H16_d128_T4"]
    B, H, d, T, steps = cfg["B"], cfg["H"], cfg["d"], cfg["T"], cfg["steps"]
    if args.decode_steps:
        steps = args.decode_steps
    pshape = cfg["prefill"]
    log(f"decode setup: seeded {pshape.L}-token fp32 prefill for {B}x{H} units")
    S0 = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    # the seeding prefill runs in batch slabs to bound host memory
    slab = 32
    for b0 in range(0, B, slab):
        sub = synth.GDNShape(slab, pshape.L, H, d, d, "head", pshape.shift, "f32")
        x = _slab_inputs(synth, pshape, b0, slab)
        t = {kk: torch.from_numpy(vv).to("cuda") for kk, vv in x.items()}
        lt2.lt2_gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"], state_out=S0[b0:b0 + slab],
                            out=torch.empty((slab, sub.L, H, d), dtype=torch.float32, device="cuda"))
        del t, x
    torch.cuda.synchronize()
    state = torch.empty((T, B, H, d, d), dtype=torch.float32, device="cuda")
    for t in range(T):
        state[t].copy_(S0)
    del S0
    log(f"decode inputs: {steps} tokens x {T} loops fresh per step")
    x = synth.decode_inputs(seed=0, B=B, H=H, T=T, steps=steps, d=d)
    dx = {kk: torch.from_numpy(vv).to("cuda") for kk, vv in x.items()}
    del x
    out = torch.empty((steps, T, B, H, d), dtype=torch.float32, device="cuda")
    desc = lt2.gdn_desc(B, 1, H, d, d, 64, lt2.LT2_F32, lt2.LT2_F32, lt2.LT2_GATE_HEAD)
    L_ = lt2.lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    calls = [(ctypes.byref(desc), P(dx["q"][s, t]), P(dx["k"][s, t]), P(dx["v"][s, t]), P(dx["alpha"][s, t]),
              P(dx["beta"][s, t]), P(state[t]), P(out[s, t]), sp) for s in range(steps) for t in range(T)]
    fn = L_.lt2_gdn_decode_step
    scratch = state[0].clone()  # warm-up launches update a scratch copy, not the measured states
    for s in range(min(steps, 4)):
        if fn(ctypes.byref(desc), P(dx["q"][s, 0]), P(dx["k"][s, 0]), P(dx["v"][s, 0]), P(dx["alpha"][s, 0]),
              P(dx["beta"][s, 0]), P(scratch), P(out[s, 0]), sp):
            raise RuntimeError("decode failed")
    torch.cuda.synchronize()
    del scratch
    # pass 1: wall clock over all (token, loop) launches
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for c in calls:
        if fn(*c):
            raise RuntimeError("decode failed")
    e1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    span_ms = e0.elapsed_time(e1)
    bytes_step = B * H * (2 * d * d * 4 + 4 * d * 4 + 8)
    n = len(calls)
    # pass 2: kernel time per launch (events around a sample of launches)
    sample = calls[: min(n, 256)]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sample]
    for c, (a, b) in zip(sample, evs):
        a.record(stream)
        fn(*c)
        b.record(stream)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    log(f"decode {n} launches: span {span_ms:.1f} ms, {span_ms / n * 1e3:.1f} us/launch, kernel {kern_ms * 1e3:.1f} us")
    return dict(B=B, H=H, d=d, T=T, tokens=steps, launches=n, bytes_per_launch=bytes_step,
                span_ms=span_ms, wall_s=wall_s, kernel_us=kern_ms * 1e3,
                gbs_span=bytes_step * n / span_ms / 1e6, gbs_kernel=bytes_step / kern_ms / 1e6,
                tokens_per_s_per_loop=B * steps * T / (span_ms / 1e3) / T)


def channel_flops_bytes(B, L, H, d, C):
    """Algorithmic work of the per-channel-gate prefill (whole path, per launch pair):
    per head-token 2*[C*(5d + 4d) + 4*d*d + C*C/6] flops (the pages' ordering makes
    each step rank 2); bytes: q, k, v, o bf16, alpha fp32 per channel, beta fp32,
    the final state."""
    ht = B * L * H
    flops = 2.0 * ht * (C * 9 * d + 4.0 * d * d + C * C / 6.0)
    path_bytes = ht * (4 * d * 2 + 4 * d + 4) + B * H * d * d * 4.0
    return flops, path_bytes


def bench_channel(args, torch, lt2, synth, reps=3):
    """Per-channel-gate prefill, B=1 H=32 L=32768 d=128, bf16 q/k/v, chunk 64."""
    cfg = synth.WORKLOADS["channel_B1_H32_L32768_d128_bf16"]
    sh, C = cfg["shape"], cfg["chunk"]
    log(f"channel inputs B={sh.B} L={sh.L} H={sh.H} d={sh.dk}")
    x = synth.gdn_inputs(sh, seed=0)
    t = dict(q=torch.from_numpy(x["q"]).to("cuda").to(torch.bfloat16),
             k=torch.from_numpy(x["k"]).to("cuda").to(torch.bfloat16),
             v=torch.from_numpy(x["v"]).to("cuda").to(torch.bfloat16),
             alpha=torch.from_numpy(x["alpha"]).to("cuda"), beta=torch.from_numpy(x["beta"]).to("cuda"))
    del x
    out = torch.empty((sh.B, sh.L, sh.H, sh.dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((sh.B, sh.H, sh.dk, sh.dv), dtype=torch.float32, device="cuda")
    desc = lt2.gdn_desc(sh.B, sh.L, sh.H, sh.dk, sh.dv, C, lt2.LT2_BF16, lt2.LT2_BF16, lt2.LT2_GATE_CHANNEL)
    ws_bytes = lt2.lt2_gdn_prefill_workspace_size(desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    L_ = lt2.lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())
    prep = (ctypes.byref(desc), P(t["q"]), P(t["k"]), P(t["alpha"]), P(t["beta"]), P(ws), ws_bytes, sp)
    scan = (ctypes.byref(desc), P(t["q"]), P(t["k"]), P(t["v"]), None, P(out), P(S), P(ws), ws_bytes, sp)
    for _ in range(1):
        L_.lt2_gdn_prefill_prepare(*prep)
        L_.lt2_gdn_prefill_scan(*scan)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in evs:
        e[0].record(stream)
        if L_.lt2_gdn_prefill_prepare(*prep):
            raise RuntimeError("channel prepare failed")
        e[1].record(stream)
        if L_.lt2_gdn_prefill_scan(*scan):
            raise RuntimeError("channel scan failed")
        e[2].record(stream)
    torch.cuda.synchronize()
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms = prep_ms + scan_ms
    flops, pbytes = channel_flops_bytes(sh.B, sh.L, sh.H, sh.dk, C)
    log(f"channel {ms:.3f} ms (prepare {prep_ms:.3f}, scan {scan_ms:.3f})")
    return dict(B=sh.B, L=sh.L, H=sh.H, d=sh.dk, C=C, ms=ms, prepare_ms=prep_ms, scan_ms=scan_ms,
                tokens_per_s_per_loop=sh.B * sh.L / (ms / 1e3), path_flops=flops, path_bytes=pbytes,
                tflops=flops / ms / 1e9, gbs=pbytes / ms / 1e6, ws_bytes=ws_bytes)


def bench_looped(args, torch, lt2, synth, reps=5, gate=False):
    """T=4 loops of the LT2-linear block, B=2 L=8192 d_model=2048 H=16 d=128
    (with ``gate``: the sigmoid output gate inside the loop)."""
    cfg = synth.WORKLOADS["looped_B2_L8192_D2048_T4"]
    sh = cfg["shape"]
    log(f"looped inputs B={sh.B} L={sh.L} D={sh.d_model} H={sh.H} d={sh.d} T={sh.T} gate={gate}")
    w = synth.loop_weights(sh, seed=0, gate=gate)
    h0 = torch.from_numpy(synth.loop_h0(sh, seed=0)).to("cuda")
    w_in = torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16)
    w_o = torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)
    h_out = torch.empty_like(h0)
    desc = lt2.loop_desc(sh.B, sh.L, sh.d_model, sh.H, sh.d, sh.T, cfg["chunk"], int(gate))
    ws_bytes = lt2.lt2_looped_mixer_workspace_size(desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    run = lambda: lt2.lt2_looped_mixer(h0, w_in, w_o, sh.H, sh.d, sh.T, chunk=cfg["chunk"], h_out=h_out,
                                       workspace=ws, out_gate=gate)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    M, D, Hd = sh.B * sh.L, sh.d_model, sh.H * sh.d
    N_in = (4 if gate else 3) * Hd + 2 * sh.H
    gemm_flops = sh.T * 2.0 * M * D * (N_in + Hd)
    C = cfg["chunk"]
    gdn_flops = sh.T * prefill_flops_bytes(sh.B, sh.L, sh.H, sh.d, C)["path_flops"]
    log(f"looped {ms:.3f} ms per call ({sh.T} loops)")
    return dict(B=sh.B, L=sh.L, d_model=D, H=sh.H, d=sh.d, T=sh.T, out_gate=gate, ms=ms,
                tokens_per_s_per_loop=M * sh.T / (ms / 1e3),
                gemm_flops=gemm_flops, gdn_flops=gdn_flops,
                tflops=(gemm_flops + gdn_flops) / ms / 1e9,
                mfma_frac=(gemm_flops + gdn_flops) / ms / 1e9 / BF16_PEAK_TFLOPS)


def swa_flops_bytes(B, L, H, d, w, out_bytes=2):
    """Algorithmic work of causal window attention: query t scores and weights
    min(t+1, w) keys, 2 d flop each for q.k and for p v; bytes are q, k, v read
    and o written once (bf16 in)."""
    keys = sum(min(t + 1, w) for t in range(L)) if L <= 1 << 16 else (
        w * (w + 1) // 2 + (L - w) * w if L >= w else L * (L + 1) // 2)
    flops = 4.0 * d * keys * B * H
    nbytes = float(B * L * H * d * (3 * 2 + out_bytes))
    return flops, nbytes


def bench_swa(args, torch, lt2, synth, reps=20):
    """Sliding-window attention B=2 L=8192 H=16 d=128, window 512, bf16 in and out."""
    sh = synth.SWA_WORKLOAD
    log(f"swa inputs B={sh.B} L={sh.L} H={sh.H} d={sh.d} window={sh.window}")
    x = synth.swa_inputs(sh, seed=0)
    q, k, v = (torch.from_numpy(x[n]).to("cuda").to(torch.bfloat16) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    for _ in range(3):
        lt2.lt2_swa_prefill(q, k, v, sh.window, out=out)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        lt2.lt2_swa_prefill(q, k, v, sh.window, out=out)
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    flops, nbytes = swa_flops_bytes(sh.B, sh.L, sh.H, sh.d, sh.window)
    log(f"swa {ms * 1e3:.1f} us, {flops / ms / 1e9:.0f} TFLOP/s, {nbytes / ms / 1e6:.0f} GB/s")
    return dict(B=sh.B, L=sh.L, H=sh.H, d=sh.d, window=sh.window, ms=ms,
                tokens_per_s=sh.B * sh.L / (ms / 1e3), flops=flops, bytes=nbytes,
                tflops=flops / ms / 1e9, mfma_frac=flops / ms / 1e9 / BF16_PEAK_TFLOPS,
                gbs=nbytes / ms / 1e6, hbm_frac=nbytes / ms / 1e6 / HBM_PEAK_GBS)


def bench_hybrid(args, torch, lt2, synth, reps=5):
    """Looped hybrid block, B=2 L=8192 d_model=2048 H=16 d=128, shared stack
    (gated-delta layer, window-512 attention layer), T=2: four layer
    applications, the depth its parity tests hold to the bf16 bar (at eight,
    the bf16 activations of the window layers reach the bar)."""
    s3 = synth.WORKLOADS["looped_B2_L8192_D2048_T4"]["shape"]
    sh = synth.LoopShape(s3.B, s3.L, s3.d_model, s3.H, s3.d, 2)
    kinds, window, C = ("gdn", "swa"), 512, 64
    log(f"hybrid inputs B={sh.B} L={sh.L} D={sh.d_model} H={sh.H} d={sh.d} T={sh.T} layers={kinds} w={window}")
    layers = []
    for i, kind in enumerate(kinds):
        w = synth.loop_weights(sh, seed=0, kind=kind, layer=i)
        layers.append((kind, torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16),
                       torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)))
    h0 = torch.from_numpy(synth.loop_h0(sh, seed=0)).to("cuda")
    h_out = torch.empty_like(h0)
    desc = lt2.hybrid_desc(sh.B, sh.L, sh.d_model, sh.H, sh.d, sh.T, list(kinds), window, C)
    ws = torch.empty(lt2.lt2_hybrid_mixer_workspace_size(desc), dtype=torch.uint8, device="cuda")
    run = lambda: lt2.lt2_hybrid_mixer(h0, layers, sh.H, sh.d, sh.T, window, chunk=C, h_out=h_out, workspace=ws)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    M, D, Hd = sh.B * sh.L, sh.d_model, sh.H * sh.d
    gemm_flops = sh.T * 2.0 * M * D * ((3 * Hd + 2 * sh.H + Hd) + (3 * Hd + Hd))
    mixer_flops = sh.T * (prefill_flops_bytes(sh.B, sh.L, sh.H, sh.d, C)["path_flops"] +
                          swa_flops_bytes(sh.B, sh.L, sh.H, sh.d, window)[0])
    log(f"hybrid {ms:.3f} ms per call ({sh.T} loops of {len(kinds)} layers)")
    return dict(B=sh.B, L=sh.L, d_model=D, H=sh.H, d=sh.d, T=sh.T, layers=list(kinds), window=window, ms=ms,
                tokens_per_s_per_loop=M * sh.T / (ms / 1e3), gemm_flops=gemm_flops, mixer_flops=mixer_flops,
                tflops=(gemm_flops + mixer_flops) / ms / 1e9,
                mfma_frac=(gemm_flops + mixer_flops) / ms / 1e9 / BF16_PEAK_TFLOPS)


def bwd_flops_bytes(B, L, H, d, C=64):
    """Work of the backward pass as built (scalar gate, chunk C): multiply-adds
    per chunk of the prepare (K K^T, Q K^T, inverse), chunk-state (K S, N R,
    K^T U), state-cotangent (P^T dO, K dS, N^T dU, Q^T dO, K^T dR) and gradient
    kernels (K S, Q S, K dS, N R, P^T dO, N^T dU, three C x d x d accumulations,
    dO U^T, dU R^T, Q K^T, K K^T, (dP o Gam) K and its transpose, two C^3
    products, E K and E^T K); bytes are the inputs q, k, v, dO (bf16), alpha,
    beta and the fp32 gradients, each once."""
    NC = (L + C - 1) // C
    cdd, ccd, ccc = C * d * d, C * C * d, C * C * C
    macs = (2 * ccd + ccc / 6) + (2 * cdd + ccd) + (3 * cdd + 2 * ccd) + (6 * cdd + 8 * ccd + 2 * ccc)
    flops = 2.0 * macs * NC * B * H
    nbytes = float(B * L * H * (4 * d * 2 + 8 + 3 * d * 4 + 8))
    return flops, nbytes


def bench_backward(args, torch, lt2, synth, reps=5):
    """Backward pass of the headline prefill workload (B4 H16 L4096 d128 bf16).
    With bf16 inputs its products run on the bf16 matrix cores, the fp32
    intermediates as hi + lo bf16 pairs (up to three instructions per product),
    so the algorithmic rate is reported without a peak fraction."""
    sh = synth.WORKLOADS["prefill_B4_H16_L4096_d128_bf16"]["shape"]
    log(f"backward inputs B={sh.B} L={sh.L} H={sh.H} d={sh.dk} bf16")
    x = synth.gdn_inputs(sh, seed=0)
    t = {kk: torch.from_numpy(vv).to("cuda") for kk, vv in x.items()}
    q, k, v = (t[n].to(torch.bfloat16) for n in ("q", "k", "v"))
    dO = torch.from_numpy(synth.grad_out(sh, seed=0)).to("cuda").to(torch.bfloat16)
    desc = lt2.gdn_desc(sh.B, sh.L, sh.H, sh.dk, sh.dv, 64, lt2.LT2_BF16, lt2.LT2_BF16, lt2.LT2_GATE_HEAD)
    ws = torch.empty(lt2.lt2_gdn_backward_workspace_size(desc), dtype=torch.uint8, device="cuda")
    run = lambda: lt2.lt2_gdn_backward(q, k, v, t["alpha"], t["beta"], dO, workspace=ws)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    flops, nbytes = bwd_flops_bytes(sh.B, sh.L, sh.H, sh.dk)
    log(f"backward {ms:.3f} ms, {flops / ms / 1e9:.1f} TFLOP/s (algorithmic)")
    return dict(B=sh.B, L=sh.L, H=sh.H, d=sh.dk, ms=ms, tokens_per_s=sh.B * sh.L / (ms / 1e3),
                flops=flops, bytes=nbytes, tflops=flops / ms / 1e9, matrix_path="bf16, fp32 intermediates as hi+lo",
                gbs=nbytes / ms / 1e6, ws_bytes=ws.numel())


def kda_bwd_flops_bytes(B, L, H, d):
    """Work of the per-channel backward as built (token adjoint, fp32 vector
    ALUs): per head-token and state element, the forward step (2 multiply-adds
    for S^T k, 2 for the update) is run twice (checkpoint pass and segment
    recompute) and the reverse step takes 10 multiply-adds (G += q dO^T, S_t dO,
    G o E, D G, dE^T k, G^T k, G v, dE y, S_{t-1} z, the G update); bytes: q, k,
    v, dO (bf16), alpha per channel and beta read, the fp32 gradients written,
    each once."""
    ht = B * L * H
    flops = 2.0 * ht * d * d * (2 * 4 + 10)
    nbytes = float(ht * (4 * d * 2 + 4 * d + 4 + 3 * d * 4 + d * 4 + 4))
    return flops, nbytes


def bench_backward_channel(args, torch, lt2, synth, reps=3):
    """Backward pass of the per-channel prefill workload (B1 H32 L32768 d128
    bf16, alpha per key channel): the token adjoint on the vector ALUs."""
    sh = synth.WORKLOADS["channel_B1_H32_L32768_d128_bf16"]["shape"]
    log(f"channel backward inputs B={sh.B} L={sh.L} H={sh.H} d={sh.dk} bf16")
    x = synth.gdn_inputs(sh, seed=0)
    t = {kk: torch.from_numpy(vv).to("cuda") for kk, vv in x.items()}
    del x
    q, k, v = (t[n].to(torch.bfloat16) for n in ("q", "k", "v"))
    dO = torch.from_numpy(synth.grad_out(sh, seed=0)).to("cuda").to(torch.bfloat16)
    desc = lt2.gdn_desc(sh.B, sh.L, sh.H, sh.dk, sh.dv, 64, lt2.LT2_BF16, lt2.LT2_BF16, lt2.LT2_GATE_CHANNEL)
    ws = torch.empty(lt2.lt2_gdn_backward_workspace_size(desc), dtype=torch.uint8, device="cuda")
    run = lambda: lt2.lt2_gdn_backward(q, k, v, t["alpha"], t["beta"], dO, workspace=ws)
    run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    flops, nbytes = kda_bwd_flops_bytes(sh.B, sh.L, sh.H, sh.dk)
    log(f"channel backward {ms:.3f} ms, {flops / ms / 1e9:.1f} TFLOP/s (vector ALUs)")
    return dict(B=sh.B, L=sh.L, H=sh.H, d=sh.dk, ms=ms, tokens_per_s=sh.B * sh.L / (ms / 1e3), flops=flops,
                bytes=nbytes, tflops=flops / ms / 1e9, valu_frac=flops / ms / 1e9 / FP32_VALU_PEAK_TFLOPS,
                path="token adjoint, fp32 vector ALUs", ws_bytes=ws.numel())


def _slab_inputs(synth, shape, b0, nb):
    """Inputs of batch rows b0..b0+nb of the decode-seeding prefill (per-unit streams)."""
    L, H, d = shape.L, shape.H, shape.dk
    out = dict(q=np.empty((nb, L, H, d), np.float32), k=np.empty((nb, L, H, d), np.float32),
               v=np.empty((nb, L, H, d), np.float32), alpha=np.empty((nb, L, H), np.float32),
               beta=np.empty((nb, L, H), np.float32))
    from concurrent.futures import ThreadPoolExecutor

    def fill(bh):
        b, h = bh
        u = synth.gdn_unit(shape, 0, b0 + b, h)
        for kk, vv in u.items():
            out[kk][b, :, h] = vv

    with ThreadPoolExecutor(16) as ex:
        list(ex.map(fill, [(b, h) for b in range(nb) for h in range(H)]))
    return out


def bench_swa_decode(args, torch, lt2, launches=32):
    """Decode step of the window mixer: 256 sequences x 16 heads, d = 128,
    window 512, full rings (position 4095), bf16 q/k/v/out; the rings are
    streamed once per launch.  Two ring sets alternate so that consecutive
    launches do not re-read the last one's from the last-level cache.  Inputs
    drawn on the device with a fixed generator."""
    B, H, d, w = 256, 16, 128, 512
    g = torch.Generator(device="cuda").manual_seed(4321)
    rings = [tuple((torch.randn((B, H, w, d), device="cuda", generator=g) * 0.1).to(torch.bfloat16)
                   for _ in range(2)) for _ in range(2)]
    q, k, v = (torch.randn((B, H, d), device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    pos = torch.full((B,), 4095, dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    for i in range(4):
        lt2.lt2_swa_decode_step(q, k, v, *rings[i % 2], pos, w, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        lt2.lt2_swa_decode_step(q, k, v, *rings[i % 2], pos, w, out=out)
        b.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
    nbytes = B * H * (2.0 * w * d * 2 + 4 * d * 2 + 2 * d * 2)   # rings read, q/k/v/o, the new slot written
    del rings
    torch.cuda.empty_cache()
    log(f"swa decode {us:.1f} us per launch ({nbytes / us / 1e3:.0f} GB/s)")
    return dict(B=B, H=H, d=d, window=w, us_per_launch=us, bytes_per_launch=nbytes, gbs=nbytes / us / 1e3,
                hbm_frac=nbytes / us / 1e3 / HBM_PEAK_GBS, tokens_per_s=B / (us / 1e6))


def bench_hybrid_decode(args, torch, lt2, steps=8):
    """Looped hybrid decode chain: 256 sequences, d_model 2048, H16 d128, the
    (gated delta, window 512) stack at T = 2 (its tested depth), one token per
    sequence per call at position 4095 (full rings); states, rings and weights
    drawn on the device with a fixed generator."""
    B, D, H, d, T, w = 256, 2048, 16, 128, 2, 512
    g = torch.Generator(device="cuda").manual_seed(999)
    layers = []
    for kind, rows in (("gdn", 3 * H * d + 2 * H), ("swa", 3 * H * d)):
        layers.append((kind, (torch.randn((rows, D), device="cuda", generator=g) / D ** 0.5).to(torch.bfloat16),
                       (torch.randn((D, H * d), device="cuda", generator=g) / D ** 0.5).to(torch.bfloat16)))
    states = torch.randn((T, 1, B, H, d, d), device="cuda", generator=g) * 0.02
    kr = (torch.randn((T, 1, B, H, w, d), device="cuda", generator=g) * 0.1).to(torch.bfloat16)
    vr = torch.randn((T, 1, B, H, w, d), device="cuda", generator=g).to(torch.bfloat16)
    pos = torch.full((B,), 4095, dtype=torch.int32, device="cuda")
    rows = torch.randn((steps + 2, B, D), device="cuda", generator=g)
    h = torch.empty((B, D), device="cuda")
    ws = torch.empty(lt2.lt2_hybrid_decode_workspace_size(lt2.hybrid_desc(B, 1, D, H, d, T, ["gdn", "swa"], w)),
                     dtype=torch.uint8, device="cuda")
    for i in range(2):
        h.copy_(rows[i])
        lt2.lt2_hybrid_decode_step(h, layers, states, kr, vr, pos, H, d, T, w, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        h.copy_(rows[2 + i])
        a.record(stream)
        lt2.lt2_hybrid_decode_step(h, layers, states, kr, vr, pos, H, d, T, w, workspace=ws)
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    weight_bytes = sum(wi.numel() + wo.numel() for _, wi, wo in layers) * 2.0
    step_bytes = T * (2.0 * B * H * d * d * 4 + 2.0 * B * H * w * d * 2 + weight_bytes)
    del layers, states, kr, vr, rows
    torch.cuda.empty_cache()
    log(f"hybrid decode {ms:.3f} ms per token step ({step_bytes / ms / 1e6:.0f} GB/s)")
    return dict(B=B, d_model=D, H=H, d=d, T=T, layers=["gdn", "swa"], window=w, ms_per_token=ms,
                tokens_per_s=B / (ms / 1e3), bytes_per_token=step_bytes, gbs=step_bytes / ms / 1e6,
                hbm_frac=step_bytes / ms / 1e6 / HBM_PEAK_GBS)


def bench_decode_flat(args, torch, lt2, launches=64):
    """Decode-step time against the context length behind the state (the pages'
    flat decode throughput): the 4096-unit state of the decode workload (256
    sequences x 16 heads, d=128) is seeded by a 2048-token and by a 32768-token
    bf16 prefill of 16 sequences (tiled to 256), then the same fp32 decode step
    is timed on each, rotating over four copies of the state.  Inputs are drawn
    on the device with a fixed generator."""
    B, H, d, Bs = 256, 16, 128, 16
    g = torch.Generator(device="cuda").manual_seed(1234)
    res = {}
    for L in (2048, 32768):
        qk = [torch.nn.functional.normalize(torch.randn((Bs, L, H, d), device="cuda", generator=g), dim=-1)
              .to(torch.bfloat16) for _ in range(2)]
        vv = torch.randn((Bs, L, H, d), device="cuda", generator=g).to(torch.bfloat16)
        a = torch.sigmoid(-torch.randn((Bs, L, H), device="cuda", generator=g))
        bt = torch.sigmoid(torch.randn((Bs, L, H), device="cuda", generator=g))
        S = torch.empty((Bs, H, d, d), dtype=torch.float32, device="cuda")
        lt2.lt2_gdn_prefill(qk[0], qk[1], vv, a, bt, state_out=S, out=torch.empty_like(vv))
        del qk, vv, a, bt
        # four copies rotated per launch, as the loops of the decode workload do, so the
        # 1 GiB of state is streamed from HBM rather than re-hit in the last-level cache
        state = S.repeat(B // Bs, 1, 1, 1).unsqueeze(0).repeat(4, 1, 1, 1, 1).contiguous()
        q = torch.nn.functional.normalize(torch.randn((B, H, d), device="cuda", generator=g), dim=-1)
        k = torch.nn.functional.normalize(torch.randn((B, H, d), device="cuda", generator=g), dim=-1)
        v = torch.randn((B, H, d), device="cuda", generator=g)
        al = torch.sigmoid(-torch.randn((B, H), device="cuda", generator=g))
        be = torch.sigmoid(torch.randn((B, H), device="cuda", generator=g))
        out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
        for i in range(4):
            lt2.lt2_gdn_decode_step(q, k, v, al, be, state[i], out=out)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        for i, (e0, e1) in enumerate(ev):
            e0.record()
            lt2.lt2_gdn_decode_step(q, k, v, al, be, state[i % 4], out=out)
            e1.record()
        torch.cuda.synchronize()
        res[L] = float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]))
        del state, S
        torch.cuda.empty_cache()
    log(f"decode flat: {res[2048]:.1f} us/launch after 2048 tokens, {res[32768]:.1f} us after 32768")
    return dict(units=B * H, d=d, us_per_launch_after_2048=res[2048], us_per_launch_after_32768=res[32768],
                ratio=res[32768] / res[2048])


def bench_looped_decode(args, torch, lt2, synth, tokens=16, warm=3):
    """Looped decode chain: 256 sequences, d_model 2048, H=16, d=128, T=4 loop
    states carried in place, one token per step (fresh seeded h rows)."""
    B, D, H, d, T = 256, 2048, 16, 128, 4
    sh = synth.LoopShape(B, 1, D, H, d, T)
    log(f"looped decode B={B} D={D} H={H} d={d} T={T}, {tokens} tokens")
    w = synth.loop_weights(sh, seed=0)
    w_in = torch.from_numpy(w["w_in"]).to("cuda").to(torch.bfloat16)
    w_o = torch.from_numpy(w["w_o"]).to("cuda").to(torch.bfloat16)
    states = torch.zeros((T, B, H, d, d), dtype=torch.float32, device="cuda")
    rows = [torch.from_numpy(synth.loop_h0(synth.LoopShape(B, 1, D, H, d, T), seed=100 + i)[:, 0]).to("cuda")
            for i in range(tokens + warm)]
    hbuf = torch.empty((B, D), dtype=torch.float32, device="cuda")
    desc = lt2.loop_desc(B, 1, D, H, d, T, 64)
    ws = torch.empty(lt2.lt2_looped_decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(warm):
        hbuf.copy_(rows[i])
        lt2.lt2_looped_decode_step(hbuf, w_in, w_o, states, H, d, T, workspace=ws)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(tokens)]
    for i in range(tokens):
        hbuf.copy_(rows[warm + i])
        ev[i][0].record(stream)
        lt2.lt2_looped_decode_step(hbuf, w_in, w_o, states, H, d, T, workspace=ws)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    state_bytes = 2.0 * T * B * H * d * d * 4
    weight_bytes = T * ((3 * H * d + 2 * H) * D + D * H * d) * 2.0
    step_bytes = state_bytes + weight_bytes + T * B * (2 * D * 4 + D * 2)
    flops = T * 2.0 * B * D * (3 * H * d + 2 * H + H * d) + T * B * H * 8.0 * d * d
    log(f"looped decode {ms:.3f} ms per token step ({step_bytes / ms / 1e6:.0f} GB/s)")
    return dict(B=B, d_model=D, H=H, d=d, T=T, tokens=tokens, ms_per_token=ms,
                tokens_per_s=B / (ms / 1e3), tokens_per_s_per_loop=B * T / (ms / 1e3),
                bytes_per_token=step_bytes, gbs=step_bytes / ms / 1e6, hbm_frac=step_bytes / ms / 1e6 / HBM_PEAK_GBS,
                flops_per_token=flops, tflops=flops / ms / 1e9)


def cpu_baseline(synth):
    """The fp64 oracle on the whole headline workload (4 sequences x 4096 tokens x
    16 heads, seed 0); tokens/s per loop = B*L / t."""
    import oracle
    shape = synth.WORKLOADS["prefill_B4_H16_L4096_d128_bf16"]["shape"]
    x = synth.gdn_inputs(shape, seed=0)
    threads = oracle.max_threads()
    # whole-workload passes repeated until at least 5 s of CPU time have elapsed
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], threads=threads)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= 5.0:
            break
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return dict(value=runs * shape.B * shape.L / dt, unit="tokens/s", cores=threads, kind="oracle",
                cpu_model=cpu_model,
                sample=f"the whole headline workload ({shape.B} x {shape.L} tokens x {shape.H} heads, "
                       f"d={shape.dk}), fp64 token-by-token recurrence, {runs} passes in {dt:.2f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-looped", action="store_true")
    ap.add_argument("--no-channel", action="store_true")
    ap.add_argument("--no-looped-decode", action="store_true")
    ap.add_argument("--no-decode-flat", action="store_true")
    ap.add_argument("--no-swa", action="store_true")
    ap.add_argument("--no-hybrid", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=0, help="decode tokens (default: the workload's 1024)")
    ap.add_argument("--probe-reps", type=int, default=5, help="timed launches per HBM probe shape")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_looped_amd import lt2, synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    lt2.lib()
    pre = bench_prefill(args, torch, lt2, synth)
    copy = bench_copy(torch, lt2, reps=args.probe_reps)
    dec = None if args.no_decode else bench_decode(args, torch, lt2, synth)
    loo = None if args.no_looped else bench_looped(args, torch, lt2, synth)
    loo_g = None if args.no_looped else bench_looped(args, torch, lt2, synth, gate=True)
    cha = None if args.no_channel else bench_channel(args, torch, lt2, synth)
    lde = None if args.no_looped_decode else bench_looped_decode(args, torch, lt2, synth)
    flat = None if (args.no_decode or args.no_decode_flat) else bench_decode_flat(args, torch, lt2)
    swa = None if args.no_swa else bench_swa(args, torch, lt2, synth)
    swd = None if args.no_swa else bench_swa_decode(args, torch, lt2)
    hyb = None if args.no_hybrid else bench_hybrid(args, torch, lt2, synth)
    hdc = None if args.no_hybrid else bench_hybrid_decode(args, torch, lt2)
    bwd = None if args.no_backward else bench_backward(args, torch, lt2, synth)
    bwc = None if (args.no_backward or args.no_channel) else bench_backward_channel(args, torch, lt2, synth)
    cpu = None if args.no_cpu else cpu_baseline(synth)

    value = pre["B"] * pre["L"] * 1 / (pre["ms_step"] / 1e3)
    dom_name = max(pre["kernels"], key=lambda n: pre["kernels"][n]["ms"])
    dom = pre["kernels"][dom_name]
    # algorithmic bytes and flops of the whole path (the method's own inputs,
    # outputs and contractions); the dominant kernel is held to them
    alg_bytes, alg_flops = pre["path_bytes"], pre["path_flops"]
    traffic = measured_traffic(dom_name)
    path_traffic = None
    t_other = [measured_traffic(n) for n in pre["kernels"]]
    if all(t is not None for t in t_other):
        path_traffic = float(sum(t_other))
    roof = dict(kernel=f"prefill {dom_name}", bound="hbm", achieved=alg_bytes / dom["ms"] / 1e6, peak=HBM_PEAK_GBS,
                unit="GB/s", frac=alg_bytes / dom["ms"] / 1e6 / HBM_PEAK_GBS, traffic=traffic,
                algorithmic_bytes=alg_bytes, algorithmic_flops=alg_flops, kernel_ms=dom["ms"],
                path=dict(ms=pre["event_ms"], achieved=alg_bytes / pre["event_ms"] / 1e6,
                          frac=alg_bytes / pre["event_ms"] / 1e6 / HBM_PEAK_GBS, traffic=path_traffic,
                          traffic_over_algorithmic=None if path_traffic is None else path_traffic / alg_bytes,
                          mfma_tflops=alg_flops / pre["event_ms"] / 1e9,
                          mfma_frac=alg_flops / pre["event_ms"] / 1e9 / BF16_PEAK_TFLOPS),
                copy_ceiling_gbs=copy["gbs"], frac_of_copy_ceiling=alg_bytes / dom["ms"] / 1e6 / copy["gbs"])
    extra = dict(
        prefill_kernels=pre["kernels"],
        prefill_path=dict(ms=pre["event_ms"], gbs=alg_bytes / pre["event_ms"] / 1e6,
                          tflops=alg_flops / pre["event_ms"] / 1e9,
                          hbm_frac=alg_bytes / pre["event_ms"] / 1e6 / HBM_PEAK_GBS),
        hbm_probes=copy,
    )
    if dec:
        extra["decode"] = dict(dec, hbm_frac_kernel=dec["gbs_kernel"] / HBM_PEAK_GBS,
                               copy_ceiling_frac_kernel=dec["gbs_kernel"] / copy["gbs"],
                               hbm_frac_span=dec["gbs_span"] / HBM_PEAK_GBS)
    if loo:
        extra["looped"] = loo
    if loo_g:
        extra["looped_output_gate"] = loo_g
    if cha:
        extra["channel_prefill"] = cha
    if lde:
        extra["looped_decode"] = lde
    if flat:
        extra["decode_flat"] = flat
    if swa:
        extra["swa_prefill"] = swa
    if swd:
        extra["swa_decode"] = dict(swd, copy_ceiling_frac=swd["gbs"] / copy["gbs"])
    if hyb:
        extra["hybrid"] = hyb
    if hdc:
        extra["hybrid_decode"] = hdc
    if bwd:
        extra["backward"] = bwd
    if bwc:
        extra["backward_channel"] = bwc
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": pre["ms_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gdn_prefill B=4 H=16 L=4096 d_k=d_v=128 bf16 qkv fp32 state chunk=64 T=1",
                   "global_batch": pre["B"], "seq_len": pre["L"], "heads": pre["H"], "d_head": pre["d"],
                   "chunk": pre["C"], "loops": 1, "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
