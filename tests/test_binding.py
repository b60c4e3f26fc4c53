"""Host-side argument checks of the Python binding (no GPU): every tensor is
checked against the shapes the call derives from q (or h) before anything
reaches the C ABI, which receives bare pointers and cannot check sizes.  Host
tensors of the right shapes are rejected as well (they are not device memory)."""
import pytest
import torch

from linear_attention_looped_amd import lt2

f32, bf16 = torch.float32, torch.bfloat16


def z(*shape, dtype=f32):
    return torch.zeros(shape, dtype=dtype)


def gdn_args(B=2, L=10, H=3, d=64, dtype=bf16, channel=False):
    return dict(q=z(B, L, H, d, dtype=dtype), k=z(B, L, H, d, dtype=dtype), v=z(B, L, H, d, dtype=dtype),
                alpha=z(B, L, H, d) if channel else z(B, L, H), beta=z(B, L, H))


@pytest.mark.parametrize("name,bad,exc", [
    ("k", z(2, 10, 3, 32, dtype=bf16), ValueError),        # wrong head size
    ("k", z(2, 10, 3, 64, dtype=f32), TypeError),          # dtype differs from q
    ("v", z(2, 9, 3, 64, dtype=bf16), ValueError),         # wrong length
    ("alpha", z(2, 10, 4), ValueError),                    # wrong head count
    ("alpha", z(2, 10, 3, 32), ValueError),                # per-channel gate of the wrong width
    ("alpha", z(2, 10, 3, dtype=bf16), TypeError),
    ("beta", z(2, 10, 3, 1), ValueError),
    ("beta", z(2, 10, 3, dtype=torch.float64), TypeError),
])
def test_prefill_input_shapes(name, bad, exc):
    a = gdn_args()
    a[name] = bad
    with pytest.raises(exc, match=name):
        lt2.lt2_gdn_prefill(**a)


@pytest.mark.parametrize("kw,exc", [
    (dict(out=z(2, 10, 3, 32)), ValueError),
    (dict(out=z(2, 10, 3, 64, dtype=torch.float16)), TypeError),
    (dict(state_in=z(2, 3, 64, 32)), ValueError),
    (dict(state_in=z(2, 3, 64, 64, dtype=bf16)), TypeError),
    (dict(state_out=z(3, 2, 64, 64)), ValueError),
    (dict(state_out=z(2, 3, 64, 64, dtype=bf16)), TypeError),
])
def test_prefill_output_and_state_shapes(kw, exc):
    with pytest.raises(exc):
        lt2.lt2_gdn_prefill(**gdn_args(), **kw)


def test_prefill_rejects_host_tensors_and_small_workspace():
    with pytest.raises(ValueError, match="device"):
        lt2.lt2_gdn_prefill(**gdn_args())
    with pytest.raises(ValueError, match="workspace holds"):
        lt2.lt2_gdn_prefill(**gdn_args(), workspace=z(16, dtype=torch.uint8))


def test_decode_shapes():
    a = dict(q=z(4, 2, 64), k=z(4, 2, 64), v=z(4, 2, 64), alpha=z(4, 2), beta=z(4, 2))
    with pytest.raises(ValueError, match="state"):
        lt2.lt2_gdn_decode_step(**a, state=z(4, 2, 64, 32))
    with pytest.raises(TypeError, match="state"):
        lt2.lt2_gdn_decode_step(**a, state=z(4, 2, 64, 64, dtype=bf16))
    with pytest.raises(ValueError, match="out"):
        lt2.lt2_gdn_decode_step(**a, state=z(4, 2, 64, 64), out=z(4, 2, 63))
    with pytest.raises(ValueError, match="alpha"):
        lt2.lt2_gdn_decode_step(**dict(a, alpha=z(4, 3)), state=z(4, 2, 64, 64))
    with pytest.raises(ValueError, match="device"):
        lt2.lt2_gdn_decode_step(**a, state=z(4, 2, 64, 64))


def test_backward_shapes():
    a = gdn_args()
    with pytest.raises(ValueError, match="d_out"):
        lt2.lt2_gdn_backward(**a, d_out=z(2, 10, 3, 32))
    with pytest.raises(ValueError, match="d_state_out"):
        lt2.lt2_gdn_backward(**a, d_out=z(2, 10, 3, 64), d_state_out=z(2, 3, 64))
    with pytest.raises(ValueError, match="state_in"):
        lt2.lt2_gdn_backward(**a, d_out=z(2, 10, 3, 64), state_in=z(1, 3, 64, 64))


def loop_args(B=2, L=8, D=256, H=2, d=64, gate=False):
    rows = (4 if gate else 3) * H * d + 2 * H
    return dict(h_in=z(B, L, D), W_in=z(rows, D, dtype=bf16), W_o=z(D, H * d, dtype=bf16), H=H, d_head=d, T=2,
                out_gate=gate)


@pytest.mark.parametrize("kw,exc,match", [
    (dict(W_in=z(3 * 128 + 4, 256, dtype=bf16)), ValueError, "W_in"),        # rows of the ungated block...
    (dict(W_o=z(128, 256, dtype=bf16)), ValueError, "W_o"),                  # ...W_o transposed
    (dict(W_o=z(256, 128)), TypeError, "W_o"),
    (dict(h_out=z(2, 8, 128)), ValueError, "h_out"),
    (dict(h_in=z(2, 8, 256, dtype=bf16)), TypeError, "h_in"),
])
def test_looped_shapes(kw, exc, match):
    a = loop_args(gate=True) if "W_in" in kw else loop_args()
    a.update(kw)
    with pytest.raises(exc, match=match):
        lt2.lt2_looped_mixer(**a)


def test_looped_decode_shapes():
    a = loop_args()
    h = z(2, 256)
    with pytest.raises(ValueError, match="states"):
        lt2.lt2_looped_decode_step(h, a["W_in"], a["W_o"], z(2, 2, 2, 64, 32), 2, 64, 2)
    with pytest.raises(ValueError, match="W_in"):
        lt2.lt2_looped_decode_step(h, a["W_in"][:-1], a["W_o"], z(2, 2, 2, 64, 64), 2, 64, 2)
    with pytest.raises(ValueError, match="device"):
        lt2.lt2_looped_decode_step(h, a["W_in"], a["W_o"], z(2, 2, 2, 64, 64), 2, 64, 2)


def test_swa_and_hybrid_shapes():
    q = z(1, 20, 2, 64, dtype=bf16)
    with pytest.raises(ValueError, match="v"):
        lt2.lt2_swa_prefill(q, q, z(1, 20, 2, 32, dtype=bf16), 8)
    with pytest.raises(ValueError, match="out"):
        lt2.lt2_swa_prefill(q, q, q, 8, out=z(1, 20, 2, 32))
    D, H, d = 256, 2, 64
    gdn = ("gdn", z(3 * H * d + 2 * H, D, dtype=bf16), z(D, H * d, dtype=bf16))
    swa_bad = ("swa", z(3 * H * d + 2 * H, D, dtype=bf16), z(D, H * d, dtype=bf16))   # window layers have no gate rows
    with pytest.raises(ValueError, match="layer 1 W_in"):
        lt2.lt2_hybrid_mixer(z(1, 8, D), [gdn, swa_bad], H, d, 2, 4)
    with pytest.raises(ValueError, match="unknown kind"):
        lt2.lt2_hybrid_mixer(z(1, 8, D), [("mlp", gdn[1], gdn[2])], H, d, 2, 4)
    with pytest.raises(ValueError, match="layers"):
        lt2.lt2_hybrid_mixer(z(1, 8, D), [], H, d, 2, 4)


def test_copy_sizes():
    with pytest.raises(ValueError):
        lt2.lt2_hbm_copy(z(8), z(4))
