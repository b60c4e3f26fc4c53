"""Seeded synthetic inputs for the gated-delta mixer.

This module only draws random numbers and rounds them; it holds none of the
mixer's own arithmetic, so both the fp64 oracle (tests) and the HIP path feed
from it without sharing any computation.

Every random stream is numpy's PCG64 keyed by ``[seed, tag, *unit]``, one stream
per independent unit (a (batch, head) pair, or a (batch, head, loop) triple for
decode).  Any single unit can therefore be regenerated on its own, which is how
parity checks at full workload size sample a few units for the oracle.

Recipe (the workloads named for the LT2 linear mixer):
  q, k  = N(0,1) rows divided by their L2 norm (per token and head)
  v     = N(0,1)
  beta  = sigmoid(N(0,1))
  alpha = exp(-softplus(N(0,1) + shift)), shift 0 or 2, one per head (scalar
          gate) or one per key channel (per-channel gate)
Inputs of bf16 workloads are rounded to bf16 (round-to-nearest-even) after
normalisation and returned as float32 arrays holding bf16 values.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

# stream tags
T_Q, T_K, T_V, T_BETA, T_ALPHA = 1, 2, 3, 4, 5
T_H0, T_WIN, T_WO, T_WG = 6, 7, 8, 9
T_DQ, T_DK, T_DV, T_DBETA, T_DALPHA = 11, 12, 13, 14, 15
T_SQ, T_SK, T_SV = 16, 17, 18
T_GO = 19


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(seed: int, tag: int, *unit: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag), *[int(u) for u in unit]])


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 result."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-valued float32 data, as uint16 (the bf16 encoding)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _unit_rows(g: np.random.Generator, n: int, d: int) -> np.ndarray:
    x = g.standard_normal((n, d), dtype=np.float32).astype(np.float64)
    nrm = np.sqrt((x * x).sum(axis=1, keepdims=True))
    return (x / nrm).astype(np.float32)


def _sigmoid64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def _exp_neg_softplus64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    sp = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
    return np.exp(-sp)


@dataclass(frozen=True)
class GDNShape:
    B: int
    L: int
    H: int
    dk: int
    dv: int
    gate: str = "head"      # "head" (alpha [B,L,H]) or "channel" (alpha [B,L,H,dk])
    shift: float = 0.0      # alpha = exp(-softplus(N(0,1) + shift))
    dtype: str = "f32"      # "f32" or "bf16" for q, k, v


def gdn_unit(shape: GDNShape, seed: int, b: int, h: int) -> dict:
    """Inputs of one (batch, head) unit: q,k [L,dk], v [L,dv], beta [L], alpha [L] or [L,dk]."""
    L, dk, dv = shape.L, shape.dk, shape.dv
    q = _unit_rows(rng(seed, T_Q, b, h), L, dk)
    k = _unit_rows(rng(seed, T_K, b, h), L, dk)
    v = rng(seed, T_V, b, h).standard_normal((L, dv), dtype=np.float32)
    beta = _sigmoid64(rng(seed, T_BETA, b, h).standard_normal(L)).astype(np.float32)
    ashape = (L,) if shape.gate == "head" else (L, dk)
    alpha = _exp_neg_softplus64(
        rng(seed, T_ALPHA, b, h).standard_normal(ashape) + shape.shift).astype(np.float32)
    if shape.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta)


def grad_out_unit(shape: GDNShape, seed: int, b: int, h: int) -> np.ndarray:
    """Output cotangent dO [L, dv] of one unit for the backward pass: N(0,1),
    rounded to bf16 for bf16 workloads."""
    x = rng(seed, T_GO, b, h).standard_normal((shape.L, shape.dv), dtype=np.float32)
    return bf16_round(x) if shape.dtype == "bf16" else x


def grad_out(shape: GDNShape, seed: int = 0) -> np.ndarray:
    """dO [B, L, H, dv], unit by unit as ``grad_out_unit``."""
    out = np.empty((shape.B, shape.L, shape.H, shape.dv), np.float32)

    def fill(bh):
        b, h = divmod(bh, shape.H)
        out[b, :, h] = grad_out_unit(shape, seed, b, h)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(shape.B * shape.H)))
    return out


def gdn_inputs(shape: GDNShape, seed: int = 0) -> dict:
    """Full token-major arrays: q,k [B,L,H,dk], v [B,L,H,dv], beta [B,L,H],
    alpha [B,L,H] (head gate) or [B,L,H,dk] (channel gate), all float32."""
    B, L, H, dk, dv = shape.B, shape.L, shape.H, shape.dk, shape.dv
    out = dict(
        q=np.empty((B, L, H, dk), np.float32),
        k=np.empty((B, L, H, dk), np.float32),
        v=np.empty((B, L, H, dv), np.float32),
        beta=np.empty((B, L, H), np.float32),
        alpha=np.empty((B, L, H) if shape.gate == "head" else (B, L, H, dk), np.float32),
    )

    def fill(bh):
        b, h = bh
        u = gdn_unit(shape, seed, b, h)
        for name, arr in u.items():
            out[name][b, :, h] = arr

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, [(b, h) for b in range(B) for h in range(H)]))
    return out


def decode_unit(seed: int, b: int, h: int, loop: int, steps: int, d: int) -> dict:
    """Fresh per-step decode inputs of one (batch, head, loop) unit:
    q,k [steps,d] unit rows, v [steps,d], beta/alpha [steps] (shift 0)."""
    q = _unit_rows(rng(seed, T_DQ, b, h, loop), steps, d)
    k = _unit_rows(rng(seed, T_DK, b, h, loop), steps, d)
    v = rng(seed, T_DV, b, h, loop).standard_normal((steps, d), dtype=np.float32)
    beta = _sigmoid64(rng(seed, T_DBETA, b, h, loop).standard_normal(steps)).astype(np.float32)
    alpha = _exp_neg_softplus64(rng(seed, T_DALPHA, b, h, loop).standard_normal(steps)).astype(np.float32)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta)


def decode_inputs(seed: int, B: int, H: int, T: int, steps: int, d: int) -> dict:
    """All decode inputs laid out [steps, T, B, H, ...] so that one (step, loop)
    slice is a contiguous [B, H, d] block."""
    out = dict(
        q=np.empty((steps, T, B, H, d), np.float32),
        k=np.empty((steps, T, B, H, d), np.float32),
        v=np.empty((steps, T, B, H, d), np.float32),
        beta=np.empty((steps, T, B, H), np.float32),
        alpha=np.empty((steps, T, B, H), np.float32),
    )

    def fill(b):
        for h in range(H):
            for t in range(T):
                u = decode_unit(seed, b, h, t, steps, d)
                for name, arr in u.items():
                    out[name][:, t, b, h] = arr

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(B)))
    return out


@dataclass(frozen=True)
class LoopShape:
    B: int
    L: int
    d_model: int
    H: int
    d: int
    T: int


def loop_weights(shape: LoopShape, seed: int = 0, gate: bool = False, kind: str = "gdn",
                 layer: int | None = None) -> dict:
    """bf16-valued weights in the [d_out, d_in] convention (y = x W^T):
    W_in [3*H*d + 2*H, d_model] = rows of W_q, W_k, W_v, W_beta, W_alpha, or with
    ``gate`` [4*H*d + 2*H, d_model] with W_g (its own stream) after W_v; the other
    rows are the same draws either way.  W_o [d_model, H*d].  Entries N(0, 1/d_in).
    A window-attention layer (``kind="swa"``) takes the W_q, W_k, W_v (and W_g)
    rows only.  ``layer`` keys the streams of one layer of a multi-layer block."""
    D, H, d = shape.d_model, shape.H, shape.d
    n_in = 3 * H * d + 2 * H
    s = 1.0 / np.sqrt(D)
    unit = () if layer is None else (layer,)
    w_in = rng(seed, T_WIN, *unit).standard_normal((n_in, D), dtype=np.float32) * np.float32(s)
    w_o = rng(seed, T_WO, *unit).standard_normal((D, H * d), dtype=np.float32) * np.float32(1.0 / np.sqrt(H * d))
    if kind == "swa":
        w_in = w_in[:3 * H * d]
    elif kind != "gdn":
        raise ValueError(kind)
    if gate:
        w_g = rng(seed, T_WG, *unit).standard_normal((H * d, D), dtype=np.float32) * np.float32(s)
        w_in = np.concatenate([w_in[:3 * H * d], w_g, w_in[3 * H * d:]], axis=0)
    return dict(w_in=bf16_round(w_in), w_o=bf16_round(w_o))


def loop_h0(shape: LoopShape, seed: int = 0, b: int | None = None, rows: int | None = None) -> np.ndarray:
    """Residual stream h_0 ~ N(0,1), bf16-valued float32, [B, L, d_model]
    (or the first ``rows`` tokens of batch row ``b`` when b is given)."""
    L = shape.L if rows is None else rows
    if b is not None:
        x = rng(seed, T_H0, b).standard_normal((shape.L, shape.d_model), dtype=np.float32)[:L]
        return bf16_round(x)
    out = np.empty((shape.B, L, shape.d_model), np.float32)
    for bb in range(shape.B):
        out[bb] = bf16_round(rng(seed, T_H0, bb).standard_normal((shape.L, shape.d_model), dtype=np.float32)[:L])
    return out


@dataclass(frozen=True)
class SWAShape:
    B: int
    L: int
    H: int
    d: int
    window: int


def swa_unit(shape: SWAShape, seed: int, b: int, h: int) -> dict:
    """q, k, v [L, d] of one (batch, head) unit of a window-attention layer:
    N(0,1) entries (the scale of x W^T for x ~ N(0,1) and W ~ N(0, 1/d_in)),
    rounded to bf16, float32 arrays."""
    L, d = shape.L, shape.d
    return {n: bf16_round(rng(seed, t, b, h).standard_normal((L, d), dtype=np.float32))
            for n, t in (("q", T_SQ), ("k", T_SK), ("v", T_SV))}


def swa_inputs(shape: SWAShape, seed: int = 0) -> dict:
    """q, k, v [B, L, H, d] bf16-valued float32 arrays, unit by unit as ``swa_unit``."""
    B, L, H, d = shape.B, shape.L, shape.H, shape.d
    out = {n: np.empty((B, L, H, d), np.float32) for n in ("q", "k", "v")}

    def fill(bh):
        b, h = divmod(bh, H)
        for n, arr in swa_unit(shape, seed, b, h).items():
            out[n][b, :, h] = arr

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(B * H)))
    return out


# Window-attention workload: the looped block's head shape at 8k context, window 512.
SWA_WORKLOAD = SWAShape(2, 8192, 16, 128, 512)


# The five workloads of the LT2 linear-mixer hot path, named by kind and sizes.
WORKLOADS = {
    "prefill_B1_L256_d64_f32": dict(kind="prefill", shape=GDNShape(1, 256, 1, 64, 64, "head", 0.0, "f32"), chunk=64, T=1),
    "prefill_B4_H16_L4096_d128_bf16": dict(kind="prefill", shape=GDNShape(4, 4096, 16, 128, 128, "head", 2.0, "bf16"), chunk=64, T=1),
    "looped_B2_L8192_D2048_T4": dict(kind="looped", shape=LoopShape(2, 8192, 2048, 16, 128, 4), chunk=64),
    "channel_B1_H32_L32768_d128_bf16": dict(kind="prefill", shape=GDNShape(1, 32768, 32, 128, 128, "channel", 2.0, "bf16"), chunk=64, T=1),
    "decode_B256_H16_d128_T4": dict(kind="decode", prefill=GDNShape(256, 2048, 16, 128, 128, "head", 0.0, "f32"),
            B=256, H=16, d=128, T=4, steps=1024, chunk=64),
}
