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
        L.lt2_looped_decode_step_noalloc.argtypes = [LD, P, P, P, P, P]
        L.lt2_looped_decode_step_noalloc.restype = S
        L.lt2_gdn_backward_workspace_size.argtypes = [GD]
        L.lt2_gdn_backward_workspace_size.restype = Z
        L.lt2_gdn_backward.argtypes = [GD] + [P] * 15 + [Z, P]
        L.lt2_gdn_backward.restype = S
        L.lt2_swa_prefill.argtypes = [ctypes.POINTER(lt2_swa_desc), P, P, P, P, P]
        L.lt2_swa_prefill.restype = S
        L.lt2_swa_decode_step.argtypes = [ctypes.POINTER(lt2_swa_desc), P, P, P, P, P, P, P, P]
        L.lt2_swa_decode_step.restype = S
        HD = ctypes.POINTER(lt2_hybrid_desc)
        L.lt2_hybrid_mixer_workspace_size.argtypes = [HD]
        L.lt2_hybrid_mixer_workspace_size.restype = Z
        L.lt2_hybrid_mixer.argtypes = [HD, P, P, P, P, P, Z, P]
        L.lt2_hybrid_mixer.restype = S
        L.lt2_hybrid_decode_workspace_size.argtypes = [HD]
        L.lt2_hybrid_decode_workspace_size.restype = Z
        L.lt2_hybrid_decode_step.argtypes = [HD, P, P, P, P, P, P, P, P, Z, P]
        L.lt2_hybrid_decode_step.restype = S
        L.lt2_hbm_copy.argtypes = [P, P, Z, P]
        L.lt2_hbm_copy.restype = S
        L.lt2_hbm_probe.argtypes = [P, P, Z, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
        L.lt2_hbm_probe.restype = S
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


def _expect(t, name: str, shape=None, dtypes=None):
    """Check a tensor argument's shape and dtype (ValueError / TypeError).  The
    device, placement and contiguity checks come afterwards, for all arguments
    together, in ``_on_device``, so every shape is checked first."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtypes is not None:
        dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
        if t.dtype not in dtypes:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")


def _on_device(device, **tensors):
    """Every given tensor (None entries skipped) is a contiguous device tensor on ``device``."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


_FLOATS = (torch.float32, torch.bfloat16)


def _dims(t, n: int, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _ws(workspace, need: int, device):
    """The caller's workspace (checked) or a fresh one; returns (tensor, bytes)."""
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None
    else:
        _expect(workspace, "workspace")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, {need} needed")
    _on_device(device, workspace=workspace)
    return workspace, nbytes


def gdn_desc(B, L, H, d_k, d_v, chunk=64, qkv_dtype=LT2_BF16, out_dtype=LT2_BF16, gate=LT2_GATE_HEAD):
    return lt2_gdn_desc(B, L, H, d_k, d_v, chunk, qkv_dtype, out_dtype, gate)


def lt2_gdn_prefill_workspace_size(desc: lt2_gdn_desc) -> int:
    return int(lib().lt2_gdn_prefill_workspace_size(ctypes.byref(desc)))


def _check_gdn_inputs(q, k, v, alpha, beta, token_dims: int):
    """Shapes shared by prefill (token_dims 3: [B,L,H]) and decode (2: [B,H])."""
    lead = _dims(q, token_dims + 1, "q")
    dk = lead[-1]
    lead = lead[:-1]
    _expect(q, "q", dtypes=_FLOATS)
    _expect(k, "k", lead + (dk,), q.dtype)
    dv = _dims(v, token_dims + 1, "v")[-1]
    _expect(v, "v", lead + (dv,), q.dtype)
    _expect(alpha, "alpha")
    if alpha.dim() == token_dims + 1:
        _expect(alpha, "alpha", lead + (dk,), torch.float32)
        gate = LT2_GATE_CHANNEL
    else:
        _expect(alpha, "alpha", lead, torch.float32)
        gate = LT2_GATE_HEAD
    _expect(beta, "beta", lead, torch.float32)
    return lead, dk, dv, gate


def lt2_gdn_prefill(q, k, v, alpha, beta, state_in=None, out=None, state_out=None, chunk: int = 64,
                    out_dtype=None, workspace=None, stream=None, return_state: bool = True):
    """Chunked gated-delta prefill.  q,k [B,L,H,d_k], v [B,L,H,d_v] (fp32 or bf16),
    alpha [B,L,H] or [B,L,H,d_k] fp32, beta [B,L,H] fp32, state_in [B,H,d_k,d_v]
    fp32 or None.  Returns (out [B,L,H,d_v], state_out [B,H,d_k,d_v] or None)."""
    (B, L, H), dk, dv, gate = _check_gdn_inputs(q, k, v, alpha, beta, 3)
    dev = q.device
    if out is None:
        out = torch.empty((B, L, H, dv), dtype=out_dtype or q.dtype, device=dev)
    _expect(out, "out", (B, L, H, dv), _FLOATS)
    if state_in is not None:
        _expect(state_in, "state_in", (B, H, dk, dv), torch.float32)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if state_out is not None:
        _expect(state_out, "state_out", (B, H, dk, dv), torch.float32)
    desc = gdn_desc(B, L, H, dk, dv, chunk, _dt(q), _dt(out), gate)
    workspace, nbytes = _ws(workspace, lt2_gdn_prefill_workspace_size(desc), dev)
    _on_device(dev, q=q, k=k, v=v, alpha=alpha, beta=beta, out=out, state_in=state_in, state_out=state_out)
    code = lib().lt2_gdn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace), nbytes,
                                 _stream(stream))
    _check("lt2_gdn_prefill", code)
    return out, state_out


def lt2_gdn_decode_step(q, k, v, alpha, beta, state, out=None, stream=None):
    """One decode token per (b, h): q,k [B,H,d_k], v [B,H,d_v], alpha [B,H] or
    [B,H,d_k], beta [B,H], state [B,H,d_k,d_v] fp32 (updated in place).  Returns out."""
    (B, H), dk, dv, gate = _check_gdn_inputs(q, k, v, alpha, beta, 2)
    dev = q.device
    _expect(state, "state", (B, H, dk, dv), torch.float32)
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    _expect(out, "out", (B, H, dv), _FLOATS)
    desc = gdn_desc(B, 1, H, dk, dv, 64, _dt(q), _dt(out), gate)
    _on_device(dev, q=q, k=k, v=v, alpha=alpha, beta=beta, state=state, out=out)
    code = lib().lt2_gdn_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(state), _ptr(out), _stream(stream))
    _check("lt2_gdn_decode_step", code)
    return out


def loop_desc(B, L, d_model, H, d_head, T, chunk=64, out_gate=0):
    return lt2_loop_desc(B, L, d_model, H, d_head, T, chunk, out_gate)


def lt2_looped_mixer_workspace_size(desc: lt2_loop_desc) -> int:
    return int(lib().lt2_looped_mixer_workspace_size(ctypes.byref(desc)))


def _w_in_rows(H: int, d_head: int, out_gate: bool, gdn: bool = True) -> int:
    return (4 if out_gate else 3) * H * d_head + (2 * H if gdn else 0)


def lt2_looped_mixer(h_in, W_in, W_o, H: int, d_head: int, T: int, chunk: int = 64, h_out=None,
                     workspace=None, stream=None, out_gate: bool = False):
    """T shared-weight loops of the LT2-linear block.  h_in [B,L,D] fp32,
    W_in [3*H*d + 2*H, D] bf16 ([4*H*d + 2*H, D] with the output gate),
    W_o [D, H*d] bf16 (weights stored [d_out, d_in], y = x W^T).  Returns
    h_out [B,L,D] fp32."""
    B, L, D = _dims(h_in, 3, "h_in")
    _expect(h_in, "h_in", dtypes=torch.float32)
    dev = h_in.device
    _expect(W_in, "W_in", (_w_in_rows(H, d_head, out_gate), D), torch.bfloat16)
    _expect(W_o, "W_o", (D, H * d_head), torch.bfloat16)
    if h_out is None:
        h_out = torch.empty_like(h_in)
    _expect(h_out, "h_out", (B, L, D), torch.float32)
    desc = loop_desc(B, L, D, H, d_head, T, chunk, int(out_gate))
    workspace, nbytes = _ws(workspace, lt2_looped_mixer_workspace_size(desc), dev)
    _on_device(dev, h_in=h_in, W_in=W_in, W_o=W_o, h_out=h_out)
    code = lib().lt2_looped_mixer(ctypes.byref(desc), _ptr(h_in), _ptr(h_out), _ptr(W_in), _ptr(W_o),
                                  _ptr(workspace), nbytes, _stream(stream))
    _check("lt2_looped_mixer", code)
    return h_out


def lt2_looped_decode_workspace_size(desc: lt2_loop_desc) -> int:
    return int(lib().lt2_looped_decode_workspace_size(ctypes.byref(desc)))


def lt2_looped_decode_step(h, W_in, W_o, states, H: int, d_head: int, T: int, workspace=None, stream=None,
                           out_gate: bool = False):
    """One decode token of the looped block for each of B sequences.  h [B,D]
    fp32 and states [T,B,H,d,d] fp32 are updated in place; W_in, W_o as for
    lt2_looped_mixer.  Returns h."""
    B, D = _dims(h, 2, "h")
    _expect(h, "h", dtypes=torch.float32)
    dev = h.device
    _expect(states, "states", (T, B, H, d_head, d_head), torch.float32)
    _expect(W_in, "W_in", (_w_in_rows(H, d_head, out_gate), D), torch.bfloat16)
    _expect(W_o, "W_o", (D, H * d_head), torch.bfloat16)
    desc = loop_desc(B, 1, D, H, d_head, T, 64, int(out_gate))
    workspace, nbytes = _ws(workspace, lt2_looped_decode_workspace_size(desc), dev)
    _on_device(dev, h=h, W_in=W_in, W_o=W_o, states=states)
    code = lib().lt2_looped_decode_step(ctypes.byref(desc), _ptr(h), _ptr(W_in), _ptr(W_o), _ptr(states),
                                        _ptr(workspace), nbytes, _stream(stream))
    _check("lt2_looped_decode_step", code)
    return h


LT2_NOALLOC_SCRATCH_BYTES = 32 << 20


def lt2_looped_decode_step_noalloc(h, W_in, W_o, states, H: int, d_head: int, T: int, stream=None,
                                   out_gate: bool = False):
    """lt2_looped_decode_step using the library's fixed device scratch array
    instead of a workspace: neither this wrapper nor the library allocates.
    h [B,D] fp32 and states [T,B,H,d,d] fp32 are updated in place.  Calls that
    may overlap on one GPU share the scratch array and race.  Returns h."""
    B, D = _dims(h, 2, "h")
    _expect(h, "h", dtypes=torch.float32)
    _expect(states, "states", (T, B, H, d_head, d_head), torch.float32)
    _expect(W_in, "W_in", (_w_in_rows(H, d_head, out_gate), D), torch.bfloat16)
    _expect(W_o, "W_o", (D, H * d_head), torch.bfloat16)
    _on_device(h.device, h=h, W_in=W_in, W_o=W_o, states=states)
    desc = loop_desc(B, 1, D, H, d_head, T, 64, int(out_gate))
    code = lib().lt2_looped_decode_step_noalloc(ctypes.byref(desc), _ptr(h), _ptr(W_in), _ptr(W_o), _ptr(states),
                                                _stream(stream))
    _check("lt2_looped_decode_step_noalloc", code)
    return h


def lt2_gdn_backward_workspace_size(desc: lt2_gdn_desc) -> int:
    return int(lib().lt2_gdn_backward_workspace_size(ctypes.byref(desc)))


def lt2_gdn_backward(q, k, v, alpha, beta, d_out, state_in=None, d_state_out=None, want_state_grad=True,
                     workspace=None, stream=None):
    """Gradients of the gated-delta prefill for the output cotangent d_out
    [B,L,H,d_v] and final-state cotangent d_state_out (or None); alpha [B,L,H]
    (scalar gate) or [B,L,H,d_k] (per-channel gate).  Returns dict(dq, dk, dv,
    dlog_alpha (alpha's shape), dbeta, d_state_in) of fp32 tensors."""
    (B, L, H), dk, dv, gate = _check_gdn_inputs(q, k, v, alpha, beta, 3)
    dev = q.device
    _expect(d_out, "d_out", (B, L, H, dv), _FLOATS)
    if state_in is not None:
        _expect(state_in, "state_in", (B, H, dk, dv), torch.float32)
    if d_state_out is not None:
        _expect(d_state_out, "d_state_out", (B, H, dk, dv), torch.float32)
    desc = gdn_desc(B, L, H, dk, dv, 64, _dt(q), _dt(d_out), gate)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, L, H, dk), **f32), dk=torch.empty((B, L, H, dk), **f32),
               dv=torch.empty((B, L, H, dv), **f32), dlog_alpha=torch.empty(tuple(alpha.shape), **f32),
               dbeta=torch.empty((B, L, H), **f32),
               d_state_in=torch.empty((B, H, dk, dv), **f32) if want_state_grad else None)
    workspace, nbytes = _ws(workspace, lt2_gdn_backward_workspace_size(desc), dev)
    _on_device(dev, q=q, k=k, v=v, alpha=alpha, beta=beta, d_out=d_out, state_in=state_in,
               d_state_out=d_state_out)
    code = lib().lt2_gdn_backward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                  _ptr(state_in), _ptr(d_out), _ptr(d_state_out), _ptr(out["dq"]),
                                  _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]),
                                  _ptr(out["d_state_in"]), _ptr(workspace), nbytes, _stream(stream))
    _check("lt2_gdn_backward", code)
    return out


def swa_desc(B, L, H, d, window, qkv_dtype=LT2_BF16, out_dtype=LT2_BF16):
    return lt2_swa_desc(B, L, H, d, window, qkv_dtype, out_dtype)


def lt2_swa_prefill(q, k, v, window: int, out=None, out_dtype=None, stream=None):
    """Causal sliding-window attention.  q, k, v [B,L,H,d] bf16; keys
    t-window+1 .. t for query t, scale 1/sqrt(d).  Returns out [B,L,H,d]
    (bf16, or ``out_dtype`` / the dtype of ``out``)."""
    B, L, H, d = _dims(q, 4, "q")
    _expect(q, "q", dtypes=_FLOATS)
    dev = q.device
    _expect(k, "k", (B, L, H, d), q.dtype)
    _expect(v, "v", (B, L, H, d), q.dtype)
    if out is None:
        out = torch.empty((B, L, H, d), dtype=out_dtype or torch.bfloat16, device=dev)
    _expect(out, "out", (B, L, H, d), _FLOATS)
    desc = swa_desc(B, L, H, d, int(window), _dt(q), _dt(out))
    _on_device(dev, q=q, k=k, v=v, out=out)
    code = lib().lt2_swa_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _stream(stream))
    _check("lt2_swa_prefill", code)
    return out


def lt2_swa_decode_step(q, k, v, k_cache, v_cache, pos, window: int, out=None, out_dtype=None, stream=None):
    """One decode token of sliding-window attention per sequence.  q, k, v
    [B,H,d] bf16 (the new token); k_cache, v_cache [B,H,window,d] bf16 rings,
    updated in place at slot pos[b] % window; pos [B] int32 on the device (the
    tokens each sequence has already seen; not advanced).  Returns out [B,H,d]
    (bf16, or ``out_dtype`` / the dtype of ``out``)."""
    B, H, d = _dims(q, 3, "q")
    _expect(q, "q", dtypes=_FLOATS)
    dev = q.device
    w = int(window)
    _expect(k, "k", (B, H, d), q.dtype)
    _expect(v, "v", (B, H, d), q.dtype)
    _expect(k_cache, "k_cache", (B, H, w, d), q.dtype)
    _expect(v_cache, "v_cache", (B, H, w, d), q.dtype)
    _expect(pos, "pos", (B,), torch.int32)
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype or torch.bfloat16, device=dev)
    _expect(out, "out", (B, H, d), _FLOATS)
    desc = swa_desc(B, 1, H, d, w, _dt(q), _dt(out))
    _on_device(dev, q=q, k=k, v=v, k_cache=k_cache, v_cache=v_cache, pos=pos, out=out)
    code = lib().lt2_swa_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(pos), _ptr(out), _stream(stream))
    _check("lt2_swa_decode_step", code)
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
    B, L, D = _dims(h_in, 3, "h_in")
    _expect(h_in, "h_in", dtypes=torch.float32)
    dev = h_in.device
    if not 1 <= len(layers) <= LT2_MAX_LAYERS:
        raise ValueError(f"a hybrid block has 1 .. {LT2_MAX_LAYERS} layers, got {len(layers)}")
    for i, (kind, w_in, w_o) in enumerate(layers):
        if kind not in _KINDS:
            raise ValueError(f"layer {i}: unknown kind {kind!r}")
        _expect(w_in, f"layer {i} W_in", (_w_in_rows(H, d_head, out_gate, kind == "gdn"), D), torch.bfloat16)
        _expect(w_o, f"layer {i} W_o", (D, H * d_head), torch.bfloat16)
    if h_out is None:
        h_out = torch.empty_like(h_in)
    _expect(h_out, "h_out", (B, L, D), torch.float32)
    desc = hybrid_desc(B, L, D, H, d_head, T, [k for k, _, _ in layers], window, chunk, out_gate)
    workspace, nbytes = _ws(workspace, lt2_hybrid_mixer_workspace_size(desc), dev)
    n = len(layers)
    w_in = (ctypes.c_void_p * n)(*[w.data_ptr() for _, w, _ in layers])
    w_o = (ctypes.c_void_p * n)(*[w.data_ptr() for _, _, w in layers])
    _on_device(dev, h_in=h_in, h_out=h_out, **{f"layer{i}_W_in": w for i, (_, w, _) in enumerate(layers)},
               **{f"layer{i}_W_o": w for i, (_, _, w) in enumerate(layers)})
    code = lib().lt2_hybrid_mixer(ctypes.byref(desc), _ptr(h_in), _ptr(h_out), ctypes.cast(w_in, ctypes.c_void_p),
                                  ctypes.cast(w_o, ctypes.c_void_p), _ptr(workspace), nbytes, _stream(stream))
    _check("lt2_hybrid_mixer", code)
    return h_out


def lt2_hybrid_decode_step(h, layers, states, k_rings, v_rings, pos, H: int, d_head: int, T: int, window: int,
                           workspace=None, stream=None, out_gate: bool = False):
    """One decode token per sequence through T loops of a shared layer stack
    (``layers`` as for lt2_hybrid_mixer).  h [B,D] fp32, states
    [T,n_gdn,B,H,d,d] fp32 and the rings [T,n_swa,B,H,window,d] bf16 are
    updated in place; pos [B] int32 on the device (not advanced).  Returns h."""
    B, D = _dims(h, 2, "h")
    _expect(h, "h", dtypes=torch.float32)
    dev = h.device
    if not 1 <= len(layers) <= LT2_MAX_LAYERS:
        raise ValueError(f"a hybrid block has 1 .. {LT2_MAX_LAYERS} layers, got {len(layers)}")
    for i, (kind, w_in, w_o) in enumerate(layers):
        if kind not in _KINDS:
            raise ValueError(f"layer {i}: unknown kind {kind!r}")
        _expect(w_in, f"layer {i} W_in", (_w_in_rows(H, d_head, out_gate, kind == "gdn"), D), torch.bfloat16)
        _expect(w_o, f"layer {i} W_o", (D, H * d_head), torch.bfloat16)
    n_gdn = sum(k == "gdn" for k, _, _ in layers)
    n_swa = len(layers) - n_gdn
    tensors = dict(h=h, pos=pos)
    _expect(pos, "pos", (B,), torch.int32)
    if n_gdn:
        _expect(states, "states", (T, n_gdn, B, H, d_head, d_head), torch.float32)
        tensors["states"] = states
    if n_swa:
        _expect(k_rings, "k_rings", (T, n_swa, B, H, int(window), d_head), torch.bfloat16)
        _expect(v_rings, "v_rings", (T, n_swa, B, H, int(window), d_head), torch.bfloat16)
        tensors.update(k_rings=k_rings, v_rings=v_rings)
    desc = hybrid_desc(B, 1, D, H, d_head, T, [k for k, _, _ in layers], int(window), 64, out_gate)
    workspace, nbytes = _ws(workspace, lt2_hybrid_decode_workspace_size(desc), dev)
    n = len(layers)
    w_in = (ctypes.c_void_p * n)(*[w.data_ptr() for _, w, _ in layers])
    w_o = (ctypes.c_void_p * n)(*[w.data_ptr() for _, _, w in layers])
    _on_device(dev, **tensors, **{f"layer{i}_W_in": w for i, (_, w, _) in enumerate(layers)},
               **{f"layer{i}_W_o": w for i, (_, _, w) in enumerate(layers)})
    code = lib().lt2_hybrid_decode_step(ctypes.byref(desc), _ptr(h), ctypes.cast(w_in, ctypes.c_void_p),
                                        ctypes.cast(w_o, ctypes.c_void_p), _ptr(states) if n_gdn else None,
                                        _ptr(k_rings) if n_swa else None, _ptr(v_rings) if n_swa else None,
                                        _ptr(pos), _ptr(workspace), nbytes, _stream(stream))
    _check("lt2_hybrid_decode_step", code)
    return h


def lt2_hybrid_decode_workspace_size(desc: lt2_hybrid_desc) -> int:
    return int(lib().lt2_hybrid_decode_workspace_size(ctypes.byref(desc)))


def lt2_hbm_copy(dst, src, stream=None):
    """Streaming device copy of src into dst (same byte size, multiple of 16)."""
    n = src.numel() * src.element_size()
    _on_device(src.device, src=src, dst=dst)
    if dst.numel() * dst.element_size() != n:
        raise ValueError(f"dst holds {dst.numel() * dst.element_size()} bytes, src {n}")
    _check("lt2_hbm_copy", lib().lt2_hbm_copy(_ptr(dst), _ptr(src), n, _stream(stream)))
    return dst


PROBE_COPY, PROBE_READ, PROBE_WRITE, PROBE_TILE_COPY = 0, 1, 2, 3


def lt2_hbm_probe(dst, src, mode: int = PROBE_COPY, blocks: int = 0, unroll: int = 4, stream=None):
    """Bandwidth probe: one streaming kernel over dst/src (same byte size, a
    multiple of 16) in the given access mode and launch shape."""
    n = dst.numel() * dst.element_size()
    _on_device(dst.device, dst=dst, src=src)
    if src is not None and src.numel() * src.element_size() != n:
        raise ValueError(f"dst holds {n} bytes, src {src.numel() * src.element_size()}")
    _check("lt2_hbm_probe", lib().lt2_hbm_probe(_ptr(dst), _ptr(src), n, int(mode), int(blocks), int(unroll),
                                                _stream(stream)))
    return dst
