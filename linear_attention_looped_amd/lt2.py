"""Thin ctypes binding of liblt2.so (the C ABI in include/lt2.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if liblt2.so is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblt2.so")

LT2_F32, LT2_BF16 = 0, 1
LT2_GATE_HEAD, LT2_GATE_CHANNEL = 0, 1
STATUS = {0: "LT2_OK", 1: "LT2_ERR_NULL", 2: "LT2_ERR_SHAPE", 3: "LT2_ERR_DTYPE",
          4: "LT2_ERR_UNSUPPORTED", 5: "LT2_ERR_WORKSPACE", 6: "LT2_ERR_ALIGN", 7: "LT2_ERR_HIP"}


class lt2_gdn_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "L", "H", "d_k", "d_v", "chunk", "qkv_dtype", "out_dtype", "gate")]


class lt2_loop_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "L", "d_model", "H", "d_head", "T", "chunk", "out_gate")]


class lt2_swa_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "L", "H", "d", "window", "qkv_dtype", "out_dtype")]


LT2_MAX_LAYERS = 8
LT2_MIXER_GDN, LT2_MIXER_SWA = 0, 1
_KINDS = {"gdn": LT2_MIXER_GDN, "swa": LT2_MIXER_SWA}


class lt2_hybrid_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "L", "d_model", "H", "d_head", "T", "chunk", "out_gate",
                                               "window", "n_layers")] + [("kinds", ctypes.c_int32 * LT2_MAX_LAYERS)]


class Lt2Error(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({status_string(code)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblt2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m linear_attention_looped_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        GD, LD = ctypes.POINTER(lt2_gdn_desc), ctypes.POINTER(lt2_loop_desc)
        L.lt2_status_string.argtypes = [S]
        L.lt2_status_string.restype = ctypes.c_char_p
        L.lt2_gdn_prefill_workspace_size.argtypes = [GD]
        L.lt2_gdn_prefill_workspace_size.restype = Z
        L.lt2_gdn_prefill.argtypes = [GD, P, P, P, P, P, P, P, P, P, Z, P]
        L.lt2_gdn_prefill.restype = S
        L.lt2_gdn_prefill_prepare.argtypes = [GD, P, P, P, P, P, Z, P]
        L.lt2_gdn_prefill_prepare.restype = S
        L.lt2_gdn_prefill_scan.argtypes = [GD, P, P, P, P, P, P, P, Z, P]
        L.lt2_gdn_prefill_scan.restype = S
        L.lt2_gdn_decode_step.argtypes = [GD, P, P, P, P, P, P, P, P]
        L.lt2_gdn_decode_step.restype = S
        L.lt2_looped_mixer_workspace_size.argtypes = [LD]
        L.lt2_looped_mixer_workspace_size.restype = Z
        L.lt2_looped_mixer.argtypes = [LD, P, P, P, P, P, Z, P]
        L.lt2_looped_mixer.restype = S
        L.lt2_looped_decode_workspace_size.argtypes = [LD]
        L.lt2_looped_decode_workspace_size.restype = Z
        L.lt2_looped_decode_step.argtypes = [LD, P, P, P, P, P, Z, P]
        L.lt2_looped_decode_step.restype = S
        L.lt2_gdn_backward_workspace_size.argtypes = [GD]
        L.lt2_gdn_backward_workspace_size.restype = Z
        L.lt2_gdn_backward.argtypes = [GD] + [P] * 15 + [Z, P]
        L.lt2_gdn_backward.restype = S
        L.lt2_swa_prefill.argtypes = [ctypes.POINTER(lt2_swa_desc), P, P, P, P, P]
        L.lt2_swa_prefill.restype = S
        HD = ctypes.POINTER(lt2_hybrid_desc)
        L.lt2_hybrid_mixer_workspace_size.argtypes = [HD]
        L.lt2_hybrid_mixer_workspace_size.restype = Z
        L.lt2_hybrid_mixer.argtypes = [HD, P, P, P, P, P, Z, P]
        L.lt2_hybrid_mixer.restype = S
        L.lt2_hbm_copy.argtypes = [P, P, Z, P]
        L.lt2_hbm_copy.restype = S
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().lt2_status_string(int(code)).decode()


def _check(fn: str, code: int):
    if code != 0:
        raise Lt2Error(fn, code)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LT2_F32
    if t.dtype == torch.bfloat16:
        return LT2_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")


def gdn_desc(B, L, H, d_k, d_v, chunk=64, qkv_dtype=LT2_BF16, out_dtype=LT2_BF16, gate=LT2_GATE_HEAD):
    return lt2_gdn_desc(B, L, H, d_k, d_v, chunk, qkv_dtype, out_dtype, gate)


def lt2_gdn_prefill_workspace_size(desc: lt2_gdn_desc) -> int:
    return int(lib().lt2_gdn_prefill_workspace_size(ctypes.byref(desc)))


def lt2_gdn_prefill(q, k, v, alpha, beta, state_in=None, out=None, state_out=None, chunk: int = 64,
                    out_dtype=None, workspace=None, stream=None, return_state: bool = True):
    """Chunked gated-delta prefill.  q,k [B,L,H,d_k], v [B,L,H,d_v] (fp32 or bf16),
    alpha [B,L,H] or [B,L,H,d_k] fp32, beta [B,L,H] fp32, state_in [B,H,d_k,d_v]
    fp32 or None.  Returns (out [B,L,H,d_v], state_out [B,H,d_k,d_v] or None)."""
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(alpha, "alpha", torch.float32)
    _need(beta, "beta", torch.float32)
    gate = LT2_GATE_CHANNEL if alpha.dim() == 4 else LT2_GATE_HEAD
    if out is None:
        out = torch.empty((B, L, H, dv), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    if state_in is not None:
        _need(state_in, "state_in", torch.float32)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    desc = gdn_desc(B, L, H, dk, dv, chunk, _dt(q), _dt(out), gate)
    ws_bytes = lt2_gdn_prefill_workspace_size(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    code = lib().lt2_gdn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace),
                                 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    _check("lt2_gdn_prefill", code)
    return out, state_out


def lt2_gdn_decode_step(q, k, v, alpha, beta, state, out=None, stream=None):
    """One decode token per (b, h): q,k [B,H,d_k], v [B,H,d_v], alpha [B,H] or
    [B,H,d_k], beta [B,H], state [B,H,d_k,d_v] fp32 (updated in place).  Returns out."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(alpha, "alpha", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(state, "state", torch.float32)
    gate = LT2_GATE_CHANNEL if alpha.dim() == 3 else LT2_GATE_HEAD
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    desc = gdn_desc(B, 1, H, dk, dv, 64, _dt(q), _dt(out), gate)
    code = lib().lt2_gdn_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(state), _ptr(out), _stream(stream))
    _check("lt2_gdn_decode_step", code)
    return out


def loop_desc(B, L, d_model, H, d_head, T, chunk=64, out_gate=0):
    return lt2_loop_desc(B, L, d_model, H, d_head, T, chunk, out_gate)


def lt2_looped_mixer_workspace_size(desc: lt2_loop_desc) -> int:
    return int(lib().lt2_looped_mixer_workspace_size(ctypes.byref(desc)))


def lt2_looped_mixer(h_in, W_in, W_o, H: int, d_head: int, T: int, chunk: int = 64, h_out=None,
                     workspace=None, stream=None, out_gate: bool = False):
    """T shared-weight loops of the LT2-linear block.  h_in [B,L,D] fp32,
    W_in [3*H*d + 2*H, D] bf16 ([4*H*d + 2*H, D] with the output gate),
    W_o [D, H*d] bf16.  Returns h_out [B,L,D] fp32."""
    B, L, D = h_in.shape
    _need(h_in, "h_in", torch.float32)
    _need(W_in, "W_in", torch.bfloat16)
    _need(W_o, "W_o", torch.bfloat16)
    if h_out is None:
        h_out = torch.empty_like(h_in)
    assert W_in.shape[0] == (4 if out_gate else 3) * H * d_head + 2 * H, W_in.shape
    desc = loop_desc(B, L, D, H, d_head, T, chunk, int(out_gate))
    ws_bytes = lt2_looped_mixer_workspace_size(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=h_in.device)
    code = lib().lt2_looped_mixer(ctypes.byref(desc), _ptr(h_in), _ptr(h_out), _ptr(W_in), _ptr(W_o),
                                  _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    _check("lt2_looped_mixer", code)
    return h_out


def lt2_looped_decode_workspace_size(desc: lt2_loop_desc) -> int:
    return int(lib().lt2_looped_decode_workspace_size(ctypes.byref(desc)))


def lt2_looped_decode_step(h, W_in, W_o, states, H: int, d_head: int, T: int, workspace=None, stream=None,
                           out_gate: bool = False):
    """One decode token of the looped block for each of B sequences.  h [B,D]
    fp32 and states [T,B,H,d,d] fp32 are updated in place; W_in, W_o as for
    lt2_looped_mixer.  Returns h."""
    B, D = h.shape
    _need(h, "h", torch.float32)
    _need(states, "states", torch.float32)
    _need(W_in, "W_in", torch.bfloat16)
    _need(W_o, "W_o", torch.bfloat16)
    assert tuple(states.shape) == (T, B, H, d_head, d_head), states.shape
    assert W_in.shape[0] == (4 if out_gate else 3) * H * d_head + 2 * H, W_in.shape
    desc = loop_desc(B, 1, D, H, d_head, T, 64, int(out_gate))
    ws_bytes = lt2_looped_decode_workspace_size(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=h.device)
    code = lib().lt2_looped_decode_step(ctypes.byref(desc), _ptr(h), _ptr(W_in), _ptr(W_o), _ptr(states),
                                        _ptr(workspace),
                                        0 if workspace is None else workspace.numel() * workspace.element_size(),
                                        _stream(stream))
    _check("lt2_looped_decode_step", code)
    return h


def lt2_gdn_backward_workspace_size(desc: lt2_gdn_desc) -> int:
    return int(lib().lt2_gdn_backward_workspace_size(ctypes.byref(desc)))


def lt2_gdn_backward(q, k, v, alpha, beta, d_out, state_in=None, d_state_out=None, want_state_grad=True,
                     workspace=None, stream=None):
    """Gradients of the gated-delta prefill (scalar gate) for the output
    cotangent d_out [B,L,H,d_v] and final-state cotangent d_state_out (or None).
    Returns dict(dq, dk, dv, dlog_alpha, dbeta, d_state_in) of fp32 tensors."""
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(alpha, "alpha", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(d_out, "d_out")
    assert alpha.dim() == 3, "the backward pass is built for the scalar gate"
    dev = q.device
    desc = gdn_desc(B, L, H, dk, dv, 64, _dt(q), _dt(d_out), LT2_GATE_HEAD)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, L, H, dk), **f32), dk=torch.empty((B, L, H, dk), **f32),
               dv=torch.empty((B, L, H, dv), **f32), dlog_alpha=torch.empty((B, L, H), **f32),
               dbeta=torch.empty((B, L, H), **f32),
               d_state_in=torch.empty((B, H, dk, dv), **f32) if want_state_grad else None)
    ws_bytes = lt2_gdn_backward_workspace_size(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    code = lib().lt2_gdn_backward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                  _ptr(state_in), _ptr(d_out), _ptr(d_state_out), _ptr(out["dq"]),
                                  _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]),
                                  _ptr(out["d_state_in"]), _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    _check("lt2_gdn_backward", code)
    return out


def swa_desc(B, L, H, d, window, qkv_dtype=LT2_BF16, out_dtype=LT2_BF16):
    return lt2_swa_desc(B, L, H, d, window, qkv_dtype, out_dtype)


def lt2_swa_prefill(q, k, v, window: int, out=None, out_dtype=None, stream=None):
    """Causal sliding-window attention.  q, k, v [B,L,H,d] bf16; keys
    t-window+1 .. t for query t, scale 1/sqrt(d).  Returns out [B,L,H,d]
    (bf16, or ``out_dtype`` / the dtype of ``out``)."""
    B, L, H, d = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
        assert tuple(t.shape) == (B, L, H, d), (n, t.shape)
    if out is None:
        out = torch.empty((B, L, H, d), dtype=out_dtype or torch.bfloat16, device=q.device)
    _need(out, "out")
    assert tuple(out.shape) == (B, L, H, d), out.shape
    desc = swa_desc(B, L, H, d, int(window), _dt(q), _dt(out))
    code = lib().lt2_swa_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _stream(stream))
    _check("lt2_swa_prefill", code)
    return out


def hybrid_desc(B, L, D, H, d_head, T, kinds, window, chunk=64, out_gate=0):
    kk = (ctypes.c_int32 * LT2_MAX_LAYERS)(*[_KINDS.get(x, x) if isinstance(x, str) else x for x in kinds])
    return lt2_hybrid_desc(B, L, D, H, d_head, T, chunk, int(out_gate), window, len(kinds), kk)


def lt2_hybrid_mixer_workspace_size(desc: lt2_hybrid_desc) -> int:
    return int(lib().lt2_hybrid_mixer_workspace_size(ctypes.byref(desc)))


def lt2_hybrid_mixer(h_in, layers, H: int, d_head: int, T: int, window: int, chunk: int = 64, h_out=None,
                     workspace=None, stream=None, out_gate: bool = False):
    """T loops of a shared stack of layers; ``layers`` is a list of (kind, W_in,
    W_o) with kind "gdn" or "swa" (bf16 weights as in include/lt2.h).
    h_in [B,L,D] fp32.  Returns h_out [B,L,D] fp32."""
    B, L, D = h_in.shape
    _need(h_in, "h_in", torch.float32)
    for kind, w_in, w_o in layers:
        _need(w_in, "W_in", torch.bfloat16)
        _need(w_o, "W_o", torch.bfloat16)
        n_in = (4 if out_gate else 3) * H * d_head + (2 * H if kind == "gdn" else 0)
        assert w_in.shape[0] == n_in, (kind, w_in.shape)
    if h_out is None:
        h_out = torch.empty_like(h_in)
    desc = hybrid_desc(B, L, D, H, d_head, T, [k for k, _, _ in layers], window, chunk, out_gate)
    ws_bytes = lt2_hybrid_mixer_workspace_size(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=h_in.device)
    n = len(layers)
    w_in = (ctypes.c_void_p * n)(*[w.data_ptr() for _, w, _ in layers])
    w_o = (ctypes.c_void_p * n)(*[w.data_ptr() for _, _, w in layers])
    code = lib().lt2_hybrid_mixer(ctypes.byref(desc), _ptr(h_in), _ptr(h_out), ctypes.cast(w_in, ctypes.c_void_p),
                                  ctypes.cast(w_o, ctypes.c_void_p), _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    _check("lt2_hybrid_mixer", code)
    return h_out


def lt2_hbm_copy(dst, src, stream=None):
    """Streaming device copy of src into dst (same byte size, multiple of 16)."""
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == n
    _check("lt2_hbm_copy", lib().lt2_hbm_copy(_ptr(dst), _ptr(src), n, _stream(stream)))
    return dst
