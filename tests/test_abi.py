"""C-ABI checks that need no GPU: the library loads, exports every function
include/lt2.h declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from linear_attention_looped_amd import lt2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    with open(os.path.join(ROOT, "include", "lt2.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lt2_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "lt2_gdn_prefill" in names and "lt2_gdn_decode_step" in names and "lt2_looped_mixer" in names
    L = lt2.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in range(8):
        assert lt2.status_string(code)
    assert lt2.status_string(99) == "unknown status"


def prefill(desc, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s_in=None, out=FAKE, s_out=None, ws=FAKE,
            ws_bytes=1 << 40):
    P = ctypes.c_void_p
    return lt2.lib().lt2_gdn_prefill(ctypes.byref(desc), P(q), P(k), P(v), P(a), P(b), P(s_in), P(out),
                                     P(s_out), P(ws), ws_bytes, None)


def good_desc(**kw):
    d = dict(B=2, L=100, H=3, d_k=128, d_v=128, chunk=64, qkv_dtype=1, out_dtype=1, gate=0)
    d.update(kw)
    return lt2.lt2_gdn_desc(*[d[n] for n, _ in lt2.lt2_gdn_desc._fields_])


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), 2), (dict(L=-5), 2), (dict(H=0), 2), (dict(d_k=0), 2),
    (dict(qkv_dtype=7), 3), (dict(out_dtype=-1), 3),
    (dict(d_k=96, d_v=96), 4), (dict(d_k=64, d_v=128), 4), (dict(chunk=48), 4), (dict(chunk=128), 4),
    (dict(gate=5), 4),
])
def test_prefill_rejects_bad_descriptor(kw, code):
    assert prefill(good_desc(**kw)) == code


def test_prefill_rejects_null_misaligned_and_small_workspace():
    d = good_desc()
    assert lt2.lib().lt2_gdn_prefill(None, None, None, None, None, None, None, None, None, None, 0, None) == 1
    assert prefill(d, q=None) == 1
    assert prefill(d, out=None) == 1
    assert prefill(d, b=None) == 1
    assert prefill(d, k=FAKE + 8) == 6
    assert prefill(d, s_in=FAKE + 4) == 6
    assert prefill(d, a=FAKE + 2) == 6
    need = lt2.lt2_gdn_prefill_workspace_size(d)
    assert need > 0
    assert prefill(d, ws=None) == 5
    assert prefill(d, ws_bytes=need - 1) == 5
    assert prefill(d, ws=FAKE + 4, ws_bytes=need) == 6


def test_launch_size_limits_are_checked_before_enqueue():
    # valid sizes whose grids would pass 2^32 threads: rejected on the host in
    # 64-bit arithmetic, not at launch time with a HIP error
    big = good_desc(B=1024, H=1024, L=1 << 20, chunk=16)
    assert prefill(big) == 2
    assert lt2.lt2_gdn_prefill_workspace_size(big) == 0
    assert bwd_call(big) == 2
    assert decode(good_desc(B=16384, H=1024, L=1)) == 2
    assert decode(good_desc(B=16383, H=1024, L=1), s=None) == 1     # just inside: reaches the pointer checks
    assert loop_call(good_loop(B=4096, L=1 << 19, H=2, chunk=16)) == 2


def test_workspace_size_of_invalid_descriptor_is_zero():
    assert lt2.lt2_gdn_prefill_workspace_size(good_desc(chunk=7)) == 0
    assert lt2.lt2_gdn_prefill_workspace_size(good_desc(L=0)) == 0


def decode(desc, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s=FAKE, out=FAKE):
    P = ctypes.c_void_p
    return lt2.lib().lt2_gdn_decode_step(ctypes.byref(desc), P(q), P(k), P(v), P(a), P(b), P(s), P(out), None)


def test_decode_validation():
    assert decode(good_desc(L=2)) == 2
    assert decode(good_desc(L=1, d_k=32, d_v=32)) == 4
    assert decode(good_desc(L=1), s=None) == 1
    assert decode(good_desc(L=1), out=FAKE + 2) == 6
    assert decode(good_desc(L=1, qkv_dtype=3)) == 3
    # an empty batch is valid and launches nothing
    assert decode(good_desc(L=1, B=0), q=None, k=None, v=None, a=None, b=None, s=None, out=None) == 0


def test_copy_validation():
    L = lt2.lib()
    P = ctypes.c_void_p
    assert L.lt2_hbm_copy(P(FAKE), P(FAKE), 0, None) == 0
    assert L.lt2_hbm_copy(None, P(FAKE), 16, None) == 1
    assert L.lt2_hbm_copy(P(FAKE), P(FAKE), 17, None) == 2
    assert L.lt2_hbm_copy(P(FAKE + 4), P(FAKE), 32, None) == 6


def test_probe_validation():
    L = lt2.lib()
    P = ctypes.c_void_p
    assert L.lt2_hbm_probe(P(FAKE), P(FAKE), 0, 0, 0, 4, None) == 0
    assert L.lt2_hbm_probe(P(FAKE), P(FAKE), 32, 4, 0, 4, None) == 4       # unknown mode
    assert L.lt2_hbm_probe(P(FAKE), None, 32, 3, 0, 4, None) == 1         # tile copy reads src
    assert L.lt2_hbm_probe(P(FAKE), P(FAKE), 32, 0, 0, 3, None) == 4       # unroll not built
    assert L.lt2_hbm_probe(P(FAKE), P(FAKE), 40, 0, 0, 4, None) == 2
    assert L.lt2_hbm_probe(P(FAKE), P(FAKE), 32, 0, -1, 4, None) == 2
    assert L.lt2_hbm_probe(P(FAKE), P(FAKE), 32, 0, 1 << 24, 4, None) == 2
    assert L.lt2_hbm_probe(P(FAKE), None, 32, 1, 0, 4, None) == 1         # reading needs src
    assert L.lt2_hbm_probe(None, P(FAKE), 32, 2, 0, 4, None) == 1
    assert L.lt2_hbm_probe(P(FAKE + 8), P(FAKE), 32, 0, 0, 4, None) == 6


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(lt2, "_lib", None)
    monkeypatch.setattr(lt2, "LIB_PATH", "/nonexistent/liblt2.so")
    with pytest.raises(RuntimeError):
        lt2.lib()


def loop_call(desc, h_in=FAKE, h_out=FAKE, w_in=FAKE, w_o=FAKE, ws=FAKE, ws_bytes=1 << 40):
    P = ctypes.c_void_p
    return lt2.lib().lt2_looped_mixer(ctypes.byref(desc), P(h_in), P(h_out), P(w_in), P(w_o), P(ws), ws_bytes, None)


def good_loop(**kw):
    d = dict(B=2, L=100, d_model=256, H=2, d_head=128, T=2, chunk=64, out_gate=0)
    d.update(kw)
    return lt2.lt2_loop_desc(*[d[n] for n, _ in lt2.lt2_loop_desc._fields_])


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), 2), (dict(T=-1), 2), (dict(H=0), 2), (dict(d_head=96), 4), (dict(chunk=8), 4),
    (dict(d_model=192), 4), (dict(H=1, d_head=64), 4), (dict(out_gate=2), 4),
])
def test_looped_rejects_bad_descriptor(kw, code):
    assert loop_call(good_loop(**kw)) == code


def test_looped_null_align_workspace():
    d = good_loop()
    assert lt2.lib().lt2_looped_mixer(None, None, None, None, None, None, 0, None) == 1
    assert loop_call(d, w_o=None) == 1
    assert loop_call(d, h_in=FAKE + 4) == 6
    need = lt2.lt2_looped_mixer_workspace_size(d)
    assert need > 0
    assert loop_call(d, ws_bytes=need - 1) == 5
    assert loop_call(d, ws=FAKE + 16, ws_bytes=need) == 6
    assert loop_call(good_loop(L=0), h_in=None, h_out=None, w_in=None, w_o=None, ws=None, ws_bytes=0) == 0


def loop_decode_call(desc, h=FAKE, w_in=FAKE, w_o=FAKE, states=FAKE, ws=FAKE, ws_bytes=1 << 40):
    P = ctypes.c_void_p
    return lt2.lib().lt2_looped_decode_step(ctypes.byref(desc), P(h), P(w_in), P(w_o), P(states), P(ws),
                                            ws_bytes, None)


def test_looped_decode_validation():
    d = good_loop(L=1)
    assert lt2.lib().lt2_looped_decode_step(None, None, None, None, None, None, 0, None) == 1
    assert loop_decode_call(good_loop(L=2)) == 2                 # one token per call
    assert lt2.lt2_looped_decode_workspace_size(good_loop(L=2)) == 0
    assert loop_decode_call(good_loop(L=1, d_head=96)) == 4
    assert loop_decode_call(d, states=None) == 1
    assert loop_decode_call(d, h=FAKE + 4) == 6
    need = lt2.lt2_looped_decode_workspace_size(d)
    assert need > 0
    assert loop_decode_call(d, ws_bytes=need - 1) == 5
    assert loop_decode_call(d, ws=FAKE + 16, ws_bytes=need) == 6
    # nothing to do: no sequences or no loops
    assert loop_decode_call(good_loop(L=1, B=0), h=None, w_in=None, w_o=None, states=None, ws=None, ws_bytes=0) == 0
    assert loop_decode_call(good_loop(L=1, T=0), h=None, w_in=None, w_o=None, states=None, ws=None, ws_bytes=0) == 0


def test_looped_decode_noalloc_validation():
    P = ctypes.c_void_p
    call = lambda d, h=FAKE, w_in=FAKE, w_o=FAKE, states=FAKE: lt2.lib().lt2_looped_decode_step_noalloc(
        ctypes.byref(d), P(h), P(w_in), P(w_o), P(states), None)
    assert lt2.lib().lt2_looped_decode_step_noalloc(None, None, None, None, None, None) == 1
    assert call(good_loop(L=2)) == 2
    assert call(good_loop(L=1, d_head=96)) == 4
    assert call(good_loop(L=1), states=None) == 1
    assert call(good_loop(L=1), w_o=FAKE + 8) == 6
    # beyond the fixed scratch array: rejected before any device call
    big = good_loop(L=1, B=2048, d_model=2048, H=16, d_head=128, out_gate=1)
    assert lt2.lt2_looped_decode_workspace_size(big) > lt2.LT2_NOALLOC_SCRATCH_BYTES
    assert call(big) == 5
    # nothing to do
    assert call(good_loop(L=1, B=0), h=None, w_in=None, w_o=None, states=None) == 0
    assert call(good_loop(L=1, T=0), h=None, w_in=None, w_o=None, states=None) == 0


def test_looped_gate_adds_workspace():
    assert lt2.lt2_looped_mixer_workspace_size(good_loop(out_gate=1)) > lt2.lt2_looped_mixer_workspace_size(good_loop())
    assert (lt2.lt2_looped_decode_workspace_size(good_loop(L=1, out_gate=1)) >
            lt2.lt2_looped_decode_workspace_size(good_loop(L=1)))


def swa_call(desc, q=FAKE, k=FAKE, v=FAKE, out=FAKE):
    P = ctypes.c_void_p
    return lt2.lib().lt2_swa_prefill(ctypes.byref(desc), P(q), P(k), P(v), P(out), None)


def good_swa(**kw):
    d = dict(B=2, L=300, H=3, d=128, window=64, qkv_dtype=1, out_dtype=1)
    d.update(kw)
    return lt2.lt2_swa_desc(*[d[n] for n, _ in lt2.lt2_swa_desc._fields_])


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), 2), (dict(L=-1), 2), (dict(H=0), 2), (dict(d=0), 2), (dict(window=0), 2), (dict(window=-3), 2),
    (dict(qkv_dtype=5), 3), (dict(out_dtype=2), 3),
    (dict(qkv_dtype=0), 4), (dict(d=96), 4), (dict(d=256), 4),
    (dict(B=65536, H=65536), 2), (dict(L=1 << 20, H=16), 2),
])
def test_swa_rejects_bad_descriptor(kw, code):
    assert swa_call(good_swa(**kw)) == code


def test_swa_null_and_alignment():
    assert lt2.lib().lt2_swa_prefill(None, None, None, None, None, None) == 1
    assert swa_call(good_swa(), k=None) == 1
    assert swa_call(good_swa(), out=FAKE + 8) == 6
    assert swa_call(good_swa(), v=FAKE + 2) == 6
    # empty inputs: nothing is read or written
    assert swa_call(good_swa(L=0), q=None, k=None, v=None, out=None) == 0
    assert swa_call(good_swa(B=0), q=None, k=None, v=None, out=None) == 0


def swa_dec_call(desc, q=FAKE, k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, pos=FAKE, out=FAKE):
    P = ctypes.c_void_p
    return lt2.lib().lt2_swa_decode_step(ctypes.byref(desc), P(q), P(k), P(v), P(kc), P(vc), P(pos), P(out), None)


@pytest.mark.parametrize("kw,code", [(dict(L=2), 2), (dict(L=0), 2), (dict(B=-1), 2), (dict(H=0), 2),
                                     (dict(window=0), 2), (dict(d=96), 4), (dict(qkv_dtype=0), 4),
                                     (dict(out_dtype=7), 3), (dict(B=1 << 20, H=1 << 12), 2)])
def test_swa_decode_rejects_bad_descriptor(kw, code):
    """The window decode step takes one token (L = 1) of bf16 q/k/v with d 64 or
    128, and at most 2^31 - 1 (b, h) workgroups; nothing is launched."""
    assert swa_dec_call(good_swa(**{"L": 1, **kw})) == code


def test_swa_decode_null_and_alignment():
    assert lt2.lib().lt2_swa_decode_step(None, None, None, None, None, None, None, None, None) == 1
    for name in ("q", "k", "v", "kc", "vc", "pos", "out"):
        assert swa_dec_call(good_swa(L=1), **{name: None}) == 1, name
    assert swa_dec_call(good_swa(L=1), kc=FAKE + 8) == 6
    assert swa_dec_call(good_swa(L=1), pos=FAKE + 2) == 6
    assert swa_dec_call(good_swa(L=1), kc=FAKE, vc=FAKE) == 2                  # one buffer as both rings
    assert swa_dec_call(good_swa(L=1), kc=FAKE, vc=FAKE + 4096) == 2           # overlapping rings
    # no sequences: nothing is read or written
    assert swa_dec_call(good_swa(L=1, B=0), q=None, k=None, v=None, kc=None, vc=None, pos=None, out=None) == 0


def hybrid_call(desc, h=FAKE, w_in=(FAKE,), w_o=(FAKE,), ws=FAKE, ws_bytes=1 << 40, arrays=True):
    P = ctypes.c_void_p
    wi = (P * len(w_in))(*w_in) if arrays else None
    wo = (P * len(w_o))(*w_o) if arrays else None
    return lt2.lib().lt2_hybrid_mixer(ctypes.byref(desc), P(h), P(h), ctypes.cast(wi, P) if wi else None,
                                      ctypes.cast(wo, P) if wo else None, P(ws), ws_bytes, None)


def good_hybrid(kinds=("gdn", "swa"), **kw):
    d = dict(B=1, L=300, D=256, H=2, d_head=128, T=2, window=64, chunk=64, out_gate=0)
    d.update(kw)
    return lt2.hybrid_desc(d["B"], d["L"], d["D"], d["H"], d["d_head"], d["T"], list(kinds), d["window"],
                           d["chunk"], d["out_gate"])


def test_hybrid_validation():
    assert lt2.lib().lt2_hybrid_mixer(None, None, None, None, None, None, 0, None) == 1
    two = dict(w_in=(FAKE, FAKE), w_o=(FAKE, FAKE))
    assert hybrid_call(good_hybrid(kinds=()), **two) == 2                       # no layers
    d9 = good_hybrid(kinds=["gdn"] * 8)
    d9.n_layers = 9
    assert hybrid_call(d9, **two) == 2                                          # too many layers
    assert hybrid_call(good_hybrid(kinds=("gdn", 7)), **two) == 4               # unknown kind
    assert hybrid_call(good_hybrid(window=0), **two) == 2                       # window layer needs w >= 1
    assert hybrid_call(good_hybrid(d_head=96), **two) == 4
    assert hybrid_call(good_hybrid(D=200), **two) == 4
    assert hybrid_call(good_hybrid(), arrays=False) == 1
    assert hybrid_call(good_hybrid(), w_in=(FAKE, 0), w_o=(FAKE, FAKE)) == 1
    assert hybrid_call(good_hybrid(), w_in=(FAKE, FAKE + 8), w_o=(FAKE, FAKE)) == 6
    need = lt2.lt2_hybrid_mixer_workspace_size(good_hybrid())
    assert need == lt2.lt2_looped_mixer_workspace_size(good_loop(B=1, L=300, d_model=256, H=2, d_head=128, T=2))
    assert hybrid_call(good_hybrid(), ws_bytes=need - 1, **two) == 5
    assert hybrid_call(good_hybrid(), ws=FAKE + 16, ws_bytes=need, **two) == 6
    assert lt2.lt2_hybrid_mixer_workspace_size(good_hybrid(kinds=())) == 0
    # a block of gated-delta layers needs no window; nothing to do for an empty batch
    assert hybrid_call(good_hybrid(kinds=("gdn",), window=0, B=0), h=0, w_in=(0,), w_o=(0,), ws=0, ws_bytes=0) == 0


def bwd_call(desc, ws_bytes=1 << 40, **kw):
    P = ctypes.c_void_p
    a = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, s_in=None, d_out=FAKE, ds_out=None, dq=FAKE, dk=FAKE,
             dv=FAKE, dla=FAKE, db=FAKE, ds_in=None, ws=FAKE)
    a.update(kw)
    return lt2.lib().lt2_gdn_backward(ctypes.byref(desc), *[P(a[n]) for n in (
        "q", "k", "v", "alpha", "beta", "s_in", "d_out", "ds_out", "dq", "dk", "dv", "dla", "db", "ds_in", "ws")],
        ws_bytes, None)


def test_backward_validation():
    # the channel gate has its own (larger) workspace: checkpoints and row partials
    need_c = lt2.lt2_gdn_backward_workspace_size(good_desc(gate=1))
    assert need_c > 0
    assert bwd_call(good_desc(gate=1), ws_bytes=need_c - 1) == 5
    assert bwd_call(good_desc(gate=1), dla=None) == 1
    assert bwd_call(good_desc(d_k=96, d_v=96)) == 4
    assert bwd_call(good_desc(B=-1)) == 2
    assert bwd_call(good_desc(), db=None) == 1
    assert bwd_call(good_desc(), d_out=None) == 1
    assert bwd_call(good_desc(), dq=FAKE + 4) == 6
    assert bwd_call(good_desc(), dla=FAKE + 2) == 6
    need = lt2.lt2_gdn_backward_workspace_size(good_desc())
    assert need > 0
    assert bwd_call(good_desc(), ws_bytes=need - 1) == 5
    assert bwd_call(good_desc(), ws=FAKE + 8, ws_bytes=need) == 6
    # the internal chunk is fixed: the workspace does not depend on desc->chunk
    assert lt2.lt2_gdn_backward_workspace_size(good_desc(chunk=16)) == need
    # nothing to do for an empty batch
    assert bwd_call(good_desc(B=0), q=None, k=None, v=None, alpha=None, beta=None, d_out=None, dq=None, dk=None,
                    dv=None, dla=None, db=None, ws=None, ws_bytes=0) == 0


def hybrid_dec_call(desc, h=FAKE, w_in=(FAKE, FAKE), w_o=(FAKE, FAKE), states=FAKE, kr=FAKE, vr=FAKE, pos=FAKE,
                    ws=FAKE, ws_bytes=1 << 40):
    P = ctypes.c_void_p
    wi = (P * len(w_in))(*w_in)
    wo = (P * len(w_o))(*w_o)
    return lt2.lib().lt2_hybrid_decode_step(ctypes.byref(desc), P(h), ctypes.cast(wi, P), ctypes.cast(wo, P),
                                            P(states), P(kr), P(vr), P(pos), P(ws), ws_bytes, None)


def test_hybrid_decode_validation():
    """The looped hybrid decode step takes one token (L = 1); every refused call
    returns before any launch."""
    assert hybrid_dec_call(good_hybrid(L=2)) == 2
    assert hybrid_dec_call(good_hybrid(L=1, window=0)) == 2
    assert hybrid_dec_call(good_hybrid(L=1), h=None) == 1
    assert hybrid_dec_call(good_hybrid(L=1), pos=None) == 1
    assert hybrid_dec_call(good_hybrid(L=1), kr=None) == 1                     # a window layer needs its rings
    assert hybrid_dec_call(good_hybrid(("gdn",), L=1), w_in=(FAKE,), w_o=(FAKE,), states=None) == 1
    assert hybrid_dec_call(good_hybrid(L=1), states=FAKE + 8) == 6
    assert hybrid_dec_call(good_hybrid(L=1), ws_bytes=16) == 5
    assert hybrid_dec_call(good_hybrid(L=1), kr=FAKE, vr=FAKE) == 2            # one buffer as both rings
    need = lt2.lib().lt2_hybrid_decode_workspace_size(ctypes.byref(good_hybrid(L=1)))
    assert need > 0 and lt2.lib().lt2_hybrid_decode_workspace_size(ctypes.byref(good_hybrid(L=2))) == 0
    assert hybrid_dec_call(good_hybrid(L=1, B=0), h=None, states=None, kr=None, vr=None, pos=None, ws=None,
                           ws_bytes=0) == 0
