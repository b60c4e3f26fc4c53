"""fp64 CPU oracle of the LT2 gated-delta mixer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
shares no code with the library: the recurrence lives in ``lt2_oracle.c`` (plain
C, fp64, token by token), the looped driver below uses numpy fp64 matrix
products plus the C recurrence.

Sources (the LT2 pages):
  * the state update S_t = Diag(alpha_t)(I - beta_t k_t k_t^T) S_{t-1}
    + beta_t k_t v_t^T -- LT2 explainer (paithon.it), section "Sostituire il
    motore", the state-update equation;
  * the looped composition h^(tau) = (F_N o ... o F_1) h^(tau-1), tau = 1..T,
    with shared weights -- same page, section "Profondita presa in prestito",
    first equation.
Readings where the pages are silent (read-out o_t = S_t^T q_t, no output scale,
per-head L2 normalisation of q and k in the looped block, beta = sigmoid,
alpha = exp(-softplus), fresh zero state in every loop) are listed with the
design notes of the repository.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lt2_oracle.c")
_LIB = os.path.join(_HERE, "liblt2_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile lt2_oracle.c with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-ffp-contract=off", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.lt2o_prefill.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, I]
        lib.lt2o_prefill.restype = I
        lib.lt2o_decode_step.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, I]
        lib.lt2o_decode_step.restype = I
        lib.lt2o_backward.argtypes = [I, I, I, I, I, I] + [P] * 14 + [I]
        lib.lt2o_backward.restype = I
        lib.lt2o_max_threads.restype = I
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().lt2o_max_threads())


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def prefill(q, k, v, alpha, beta, S0=None, threads: int = 0):
    """Token-by-token gated delta rule over [B, L, H, *] inputs.

    Returns (o [B,L,H,d_v], S_final [B,H,d_k,d_v]) in fp64.  alpha is [B,L,H]
    (scalar gate per head) or [B,L,H,d_k] (per-channel gate)."""
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, L, H) and beta.shape == (B, L, H)
    channel = 1 if alpha.ndim == 4 else 0
    assert alpha.shape == ((B, L, H, dk) if channel else (B, L, H))
    S0 = None if S0 is None else _f64(S0)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, L, H, dv), np.float64)
    S = np.empty((B, H, dk, dv), np.float64)
    rc = _load().lt2o_prefill(B, L, H, dk, dv, channel, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                              _ptr(beta), _ptr(S0), _ptr(o), _ptr(S), int(threads))
    if rc != 0:
        raise RuntimeError("lt2o_prefill failed")
    return o, S


def decode_step(q, k, v, alpha, beta, S, threads: int = 0):
    """One token for every unit: q,k [B,H,d_k], v [B,H,d_v], alpha [B,H] or
    [B,H,d_k], beta [B,H], S [B,H,d_k,d_v].  Returns (o, S_new) in fp64."""
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    S = _f64(S).copy()
    B, H, dk = q.shape
    dv = v.shape[-1]
    channel = 1 if alpha.ndim == 3 else 0
    o = np.empty((B, H, dv), np.float64)
    rc = _load().lt2o_decode_step(B, H, dk, dv, channel, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                  _ptr(beta), _ptr(S), _ptr(o), int(threads))
    if rc != 0:
        raise RuntimeError("lt2o_decode_step failed")
    return o, S


def backward(q, k, v, alpha, beta, dO, S0=None, dSL=None, threads: int = 0):
    """Gradients of loss = sum <dO, o> + <dS_L, S_L> through the token recurrence
    (the state-update equation of "Sostituire il motore", read out o_t = S_t^T q_t).

    Returns dict(dq, dk, dv, dlog_alpha, dbeta, dS0) in fp64; dlog_alpha is the
    gradient with respect to log alpha (alpha's shape)."""
    q, k, v, alpha, beta, dO = map(_f64, (q, k, v, alpha, beta, dO))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    channel = 1 if alpha.ndim == 4 else 0
    S0 = None if S0 is None else _f64(S0)
    dSL = None if dSL is None else _f64(dSL)
    out = dict(dq=np.empty_like(q), dk=np.empty_like(k), dv=np.empty_like(v),
               dlog_alpha=np.empty_like(alpha), dbeta=np.empty_like(beta),
               dS0=np.empty((B, H, dk, dv), np.float64))
    rc = _load().lt2o_backward(B, L, H, dk, dv, channel, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(S0), _ptr(dO), _ptr(dSL), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                               _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]), _ptr(out["dS0"]), int(threads))
    if rc != 0:
        raise RuntimeError("lt2o_backward failed")
    return out


# ---- looped LT2-linear mixer ------------------------------------------------

def _l2norm_heads(x: np.ndarray, H: int, d: int, eps: float = 1e-6) -> np.ndarray:
    """Per-head L2 normalisation x / max(||x||_2, eps) over the last d entries."""
    M = x.shape[0]
    xh = x.reshape(M, H, d)
    n = np.sqrt((xh * xh).sum(axis=-1, keepdims=True))
    return (xh / np.maximum(n, eps)).reshape(M, H * d)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _softplus(z):
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def looped_layer(h, w_in, w_o, H: int, d: int, threads: int = 0, gate: bool = False):
    """One loop iteration of the LT2-linear block on a residual stream h [B,L,D]:

        z = h W_in^T;  q,k,v(,z_g),z_beta,z_alpha = split(z)
        q, k <- per-head L2 normalisation;  beta = sigmoid(z_beta);
        alpha = exp(-softplus(z_alpha));  o = GDN(q,k,v,alpha,beta; S_0 = 0)
        gate (LT2 explainer, the sigmoid output gate inside the loop):
            o <- o * sigmoid(z_g), elementwise, one gate per channel of each head
        h <- h + o W_o^T

    W_in is [3*H*d + 2*H, D] (rows of W_q, W_k, W_v, W_beta, W_alpha) or, with
    the gate, [4*H*d + 2*H, D] (W_g after W_v); W_o is [D, H*d].  fp64."""
    h = _f64(h)
    B, L, D = h.shape
    hd = H * d
    x = h.reshape(B * L, D)
    z = x @ _f64(w_in).T
    q = _l2norm_heads(z[:, 0:hd], H, d)
    k = _l2norm_heads(z[:, hd:2 * hd], H, d)
    v = z[:, 2 * hd:3 * hd]
    gb = 4 * hd if gate else 3 * hd   # first gate-transform column
    beta = _sigmoid(z[:, gb:gb + H])
    alpha = np.exp(-_softplus(z[:, gb + H:gb + 2 * H]))
    o, _ = prefill(q.reshape(B, L, H, d), k.reshape(B, L, H, d), v.reshape(B, L, H, d),
                   alpha.reshape(B, L, H), beta.reshape(B, L, H), None, threads)
    o = o.reshape(B * L, hd)
    if gate:
        o = o * _sigmoid(z[:, 3 * hd:4 * hd])
    return h + (o @ _f64(w_o).T).reshape(B, L, D)


def looped_mixer(h0, w_in, w_o, H: int, d: int, T: int, threads: int = 0, gate: bool = False):
    """T loops of ``looped_layer`` with the same weights, h^(tau) = F(h^(tau-1))."""
    h = _f64(h0)
    for _ in range(T):
        h = looped_layer(h, w_in, w_o, H, d, threads, gate)
    return h


# ---- sliding-window attention and the GDN/SWA hybrid ------------------------
#
# Sources: the LT2 explainer (paithon.it), section "Sostituire il motore": the
# second (sparse) family lets each token attend only to a window of the w most
# recent positions; section "Il giro trasforma il calcolo in contesto": a window
# of width w applied T times reaches O(T w) tokens back.  The LT2 summary page
# (hybrid strategies figure) interleaves the two mixer kinds across depth and
# iterations.  Readings where the pages are silent: softmax attention with the
# 1/sqrt(d) scale over keys j in [t - w + 1, t] (the token itself included), no
# normalisation of q and k in the window layer, and the shared block of the
# hybrid being a fixed stack of mixer layers applied in order, each with its
# own weights, repeated T times.

def swa(q, k, v, window: int):
    """Causal sliding-window softmax attention, one query row at a time.

    q, k, v [B, L, H, d]; output o [B, L, H, d] in fp64 with
        o_t = sum_{j=max(0,t-w+1)}^{t} softmax_j(q_t . k_j / sqrt(d)) v_j
    for every batch entry and head."""
    q, k, v = map(_f64, (q, k, v))
    B, L, H, d = q.shape
    assert k.shape == q.shape and v.shape[:3] == (B, L, H) and window >= 1
    o = np.empty(v.shape, np.float64)
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        for t in range(L):
            j0 = max(0, t - window + 1)
            kw = k[b, j0:t + 1]                      # [n, H, d]
            vw = v[b, j0:t + 1]                      # [n, H, dv]
            s = np.einsum("hd,nhd->hn", q[b, t], kw) * scale
            s = s - s.max(axis=1, keepdims=True)     # the softmax is shift invariant
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            o[b, t] = np.einsum("hn,nhe->he", p, vw)
    return o


def swa_decode_step(q, k, v, k_cache, v_cache, pos, window: int):
    """One decode token of causal sliding-window attention, per sequence, with
    the window held as a ring of the last w keys and values.

    q, k, v [B, H, d]; k_cache, v_cache [B, H, w, d] (updated in place, fp64);
    pos [B] = tokens each sequence has already seen.  The new key and value go
    to ring slot pos mod w; the query then attends to every filled slot, which
    are the tokens max(0, pos-w+1) .. pos:
        o = sum_j softmax_j(q . k_j / sqrt(d)) v_j
    (the softmax does not depend on the order of the slots).  Returns o
    [B, H, d] fp64."""
    q, k, v = map(_f64, (q, k, v))
    B, H, d = q.shape
    assert k_cache.shape[:2] == (B, H) and k_cache.shape[2] == window and window >= 1
    o = np.empty((B, H, v.shape[2]), np.float64)
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        p = int(pos[b])
        slot = p % window
        k_cache[b, :, slot] = k[b]
        v_cache[b, :, slot] = v[b]
        n = min(p + 1, window)                       # filled slots: 0 .. n-1
        for h in range(H):
            s = k_cache[b, h, :n] @ q[b, h] * scale  # [n]
            e = np.exp(s - s.max())
            o[b, h] = (e / e.sum()) @ v_cache[b, h, :n]
    return o


def swa_layer(h, w_in, w_o, H: int, d: int, window: int, gate: bool = False):
    """One window-attention layer of the looped hybrid on h [B,L,D]:

        z = h W_in^T;  q, k, v (, z_g) = split(z);  o = swa(q, k, v; w)
        gate: o <- o * sigmoid(z_g);  h <- h + o W_o^T

    W_in is [3*H*d, D] (rows of W_q, W_k, W_v) or [4*H*d, D] with the gate;
    W_o is [D, H*d].  fp64."""
    h = _f64(h)
    B, L, D = h.shape
    hd = H * d
    z = h.reshape(B * L, D) @ _f64(w_in).T
    q, k, v = (z[:, i * hd:(i + 1) * hd].reshape(B, L, H, d) for i in range(3))
    o = swa(q, k, v, window).reshape(B * L, hd)
    if gate:
        o = o * _sigmoid(z[:, 3 * hd:4 * hd])
    return h + (o @ _f64(w_o).T).reshape(B, L, D)


def hybrid_mixer(h0, layers, H: int, d: int, T: int, window: int, threads: int = 0, gate: bool = False):
    """T loops of a shared block whose layers run in order; ``layers`` is a list
    of (kind, W_in, W_o) with kind "gdn" (``looped_layer``) or "swa"
    (``swa_layer``)."""
    h = _f64(h0)
    for _ in range(T):
        for kind, w_in, w_o in layers:
            if kind == "gdn":
                h = looped_layer(h, w_in, w_o, H, d, threads, gate)
            elif kind == "swa":
                h = swa_layer(h, w_in, w_o, H, d, window, gate)
            else:
                raise ValueError(kind)
    return h
