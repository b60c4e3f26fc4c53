"""Pins of the oracle's sliding-window attention and of the GDN/SWA hybrid block.

Sources: the LT2 explainer (paithon.it), section "Sostituire il motore" (the
sparse family: each token sees a window of the w most recent positions) and
section "Il giro trasforma il calcolo in contesto" (a window of width w
iterated T times reaches O(T w) tokens back); the LT2 summary page's figure of
hybrid strategies (mixers interleaved across depth and iterations).

The pages print no worked example, so the window attention is pinned against a
library routine (torch's scaled_dot_product_attention in float64, causal or
with a band mask), closed forms (window 1, zero queries, a dominant key) and
exact invariants (which outputs a perturbed value or input can reach, shift
invariance of the scores).  A wrong window edge, a missing scale, a softmax
over the wrong axis or an off-by-one in the loop composition fails one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_looped_amd import synth


def rand_qkv(seed, B, L, H, d):
    g = np.random.default_rng(seed)
    return tuple(g.standard_normal((B, L, H, d)) for _ in range(3))


def torch_attention(q, k, v, mask=None, causal=False):
    """torch's fused attention in float64 on [B,L,H,d] arrays."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal)
    return o.numpy().transpose(0, 2, 1, 3)


@pytest.mark.parametrize("L,w", [(1, 1), (7, 7), (12, 40)])
def test_full_window_is_causal_attention(L, w):
    q, k, v = rand_qkv(1, 2, L, 3, 5)
    np.testing.assert_allclose(oracle.swa(q, k, v, w), torch_attention(q, k, v, causal=True),
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("L,w", [(9, 2), (16, 5), (33, 8)])
def test_band_matches_masked_library_attention(L, w):
    q, k, v = rand_qkv(2, 1, L, 2, 4)
    t = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    band = (j <= t) & (j > t - w)
    np.testing.assert_allclose(oracle.swa(q, k, v, w), torch_attention(q, k, v, mask=band),
                               rtol=0, atol=1e-13)


def test_window_one_returns_the_values():
    q, k, v = rand_qkv(3, 2, 11, 2, 6)
    assert np.array_equal(oracle.swa(q, k, v, 1), v)


@pytest.mark.parametrize("w", [1, 3, 6, 50])
def test_zero_queries_average_the_window(w):
    _, k, v = rand_qkv(4, 1, 20, 2, 3)
    q = np.zeros_like(k)
    c = np.concatenate([np.zeros((1, 1, 2, 3)), np.cumsum(v, axis=1)], axis=1)
    t = np.arange(20)
    lo = np.maximum(0, t - w + 1)
    mean = (c[:, t + 1] - c[:, lo]) / (t + 1 - lo)[None, :, None, None]
    np.testing.assert_allclose(oracle.swa(q, k, v, w), mean, rtol=0, atol=1e-14)


def test_dominant_key_is_seen_exactly_inside_its_window():
    L, w, d, m = 24, 5, 4, 7
    e = np.zeros(d)
    e[0] = 1.0
    q = np.broadcast_to(e, (1, L, 1, d)).copy()
    k = np.zeros((1, L, 1, d))
    k[0, m, 0] = 200.0 * np.sqrt(d) * e        # score 200 against 0 for every other key
    v = np.random.default_rng(5).standard_normal((1, L, 1, d))
    o = oracle.swa(q, k, v, w)
    for t in range(L):
        lo = max(0, t - w + 1)
        if lo <= m <= t:
            np.testing.assert_allclose(o[0, t, 0], v[0, m, 0], rtol=0, atol=1e-12)
        else:
            np.testing.assert_allclose(o[0, t, 0], v[0, lo:t + 1, 0].mean(axis=0), rtol=0, atol=1e-13)


@pytest.mark.parametrize("w", [1, 4, 9])
def test_a_value_reaches_exactly_the_next_w_outputs(w):
    q, k, v = rand_qkv(6, 1, 20, 2, 3)
    j = 8
    v2 = v.copy()
    v2[0, j] += 1.0
    diff = np.abs(oracle.swa(q, k, v2, w) - oracle.swa(q, k, v, w)).max(axis=(2, 3))[0]
    inside = (np.arange(20) >= j) & (np.arange(20) <= j + w - 1)
    assert np.all(diff[~inside] == 0.0)
    assert np.all(diff[inside] > 1e-6)


def test_scores_shift_invariance_and_scale():
    q, k, v = rand_qkv(7, 1, 15, 2, 8)
    u = np.random.default_rng(8).standard_normal(8)
    # adding one vector to every key shifts each query's scores by a constant
    np.testing.assert_allclose(oracle.swa(q, k + u, v, 6), oracle.swa(q, k, v, 6), rtol=0, atol=1e-12)
    # the 1/sqrt(d) scale: duplicating every channel (keys scaled by 1/sqrt 2) leaves the scores as they were
    q2 = np.concatenate([q, q], axis=-1)
    k2 = np.concatenate([k, k], axis=-1) / np.sqrt(2.0)
    np.testing.assert_allclose(oracle.swa(q2, k2, v, 6), oracle.swa(q, k, v, 6), rtol=0, atol=1e-12)


def test_window_edges_batch_and_heads_are_independent():
    q, k, v = rand_qkv(9, 3, 10, 4, 3)
    o = oracle.swa(q, k, v, 4)
    for b in range(3):
        for h in range(4):
            ob = oracle.swa(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1], 4)
            assert np.array_equal(ob[0, :, 0], o[b, :, h])


# ---- hybrid block -------------------------------------------------------------

def hybrid_case(kinds, gate=False, seed=21, B=1, L=14, D=8, H=2, d=3):
    shape = synth.LoopShape(B, L, D, H, d, 1)
    layers = []
    for i, kind in enumerate(kinds):
        w = synth.loop_weights(shape, seed, gate, kind=kind, layer=i)
        layers.append((kind, w["w_in"], w["w_o"]))
    h0 = np.random.default_rng(seed).standard_normal((B, L, D))
    return shape, layers, h0


def test_gdn_only_block_is_the_looped_mixer():
    shape, layers, h0 = hybrid_case(["gdn"])
    _, w_in, w_o = layers[0]
    np.testing.assert_array_equal(oracle.hybrid_mixer(h0, layers, 2, 3, 3, window=4),
                                  oracle.looped_mixer(h0, w_in, w_o, 2, 3, 3))


def test_hybrid_block_is_the_composition_of_its_layers():
    _, layers, h0 = hybrid_case(["gdn", "swa"], gate=True)
    h = h0
    for _ in range(2):
        h = oracle.looped_layer(h, layers[0][1], layers[0][2], 2, 3, gate=True)
        h = oracle.swa_layer(h, layers[1][1], layers[1][2], 2, 3, 4, gate=True)
    np.testing.assert_array_equal(oracle.hybrid_mixer(h0, layers, 2, 3, 2, window=4, gate=True), h)


def test_swa_layer_with_zero_value_or_output_weights_is_identity():
    _, layers, h0 = hybrid_case(["swa"])
    _, w_in, w_o = layers[0]
    w_in0 = w_in.copy()
    w_in0[12:18] = 0.0                               # W_v rows (H*d = 6: q, k, v blocks of 6)
    assert np.array_equal(oracle.swa_layer(h0, w_in0, w_o, 2, 3, 4), h0)
    assert np.array_equal(oracle.swa_layer(h0, w_in, np.zeros_like(w_o), 2, 3, 4), h0)


def test_swa_layer_gate_with_zero_weights_halves_the_output():
    _, layers, h0 = hybrid_case(["swa"], gate=True)
    _, w_in, w_o = layers[0]
    w_in0 = w_in.copy()
    w_in0[18:24] = 0.0                               # all of W_g: sigmoid(0) = 1/2
    plain = oracle.swa_layer(h0, w_in0[:18], w_o, 2, 3, 4)
    np.testing.assert_allclose(oracle.swa_layer(h0, w_in0, w_o, 2, 3, 4, gate=True) - h0,
                               0.5 * (plain - h0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("T,w", [(1, 3), (2, 3), (3, 4)])
def test_receptive_field_of_the_looped_window_block_is_T_times_w(T, w):
    """A change of token j's input reaches, after T loops of a window-w layer,
    exactly the tokens j .. j + T (w - 1): each loop carries it w - 1 further."""
    L = 24
    _, layers, h0 = hybrid_case(["swa"], L=L)
    j = 5
    h1 = h0.copy()
    h1[0, j] += 0.5
    diff = np.abs(oracle.hybrid_mixer(h1, layers, 2, 3, T, window=w)
                  - oracle.hybrid_mixer(h0, layers, 2, 3, T, window=w)).max(axis=2)[0]
    t = np.arange(L)
    inside = (t >= j) & (t <= j + T * (w - 1))
    assert np.all(diff[~inside] == 0.0)
    assert np.all(diff[inside] > 0.0)


# ---- decode form: the window as a ring of the last w keys and values ----

def decode_chain(q, k, v, w, start=None):
    """oracle.swa_decode_step applied token by token from empty rings."""
    B, L, H, d = q.shape
    kc, vc = np.zeros((B, H, w, d)), np.zeros((B, H, w, d))
    out = np.empty((B, L, H, d))
    for t in range(L):
        out[:, t] = oracle.swa_decode_step(q[:, t], k[:, t], v[:, t], kc, vc, np.full(B, t), w)
    return out


@pytest.mark.parametrize("L,w", [(9, 1), (20, 3), (20, 8), (13, 30)])
def test_decode_chain_is_window_attention(L, w):
    """Token-by-token decode through the ring equals torch's banded attention
    (and the oracle's prefill) at every token, across the ring's wrap-around."""
    q, k, v = rand_qkv(5, 2, L, 3, 6)
    got = decode_chain(q, k, v, w)
    i = np.arange(L)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - w)
    mask = np.where(band, 0.0, -np.inf)
    np.testing.assert_allclose(got, torch_attention(q, k, v, mask=mask), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, oracle.swa(q, k, v, w), rtol=1e-12, atol=1e-12)


def test_decode_window_one_returns_v():
    q, k, v = rand_qkv(6, 2, 5, 2, 4)
    np.testing.assert_array_equal(decode_chain(q, k, v, 1), v)


def test_decode_ring_order_and_positions():
    """A full ring whose slots are permuted gives the same output (the softmax
    ignores slot order); a sequence that has seen p < w - 1 tokens attends only
    to slots 0 .. p, whatever the other slots hold."""
    g = np.random.default_rng(7)
    B, H, w, d = 2, 3, 6, 4
    kc, vc = g.standard_normal((B, H, w, d)), g.standard_normal((B, H, w, d))
    q, k, v = (g.standard_normal((B, H, d)) for _ in range(3))
    pos = np.array([13, 2])
    o = oracle.swa_decode_step(q, k, v, kc.copy(), vc.copy(), pos, w)
    perm = g.permutation(w)                       # slot s of the permuted ring holds slot perm[s]
    kp, vp = kc[:, :, perm].copy(), vc[:, :, perm].copy()
    s1 = int(np.argsort(perm)[13 % w])            # where the slot the new token replaces went
    op = oracle.swa_decode_step(q[:1], k[:1], v[:1], kp[:1], vp[:1], np.array([w + s1]), w)
    np.testing.assert_allclose(op[0], o[0], rtol=1e-12, atol=1e-12)
    kz, vz = kc.copy(), vc.copy()
    kz[1, :, 3:], vz[1, :, 3:] = 1e3, -1e3        # unfilled slots of sequence 1
    oz = oracle.swa_decode_step(q, k, v, kz, vz, pos, w)
    np.testing.assert_allclose(oz[1], o[1], rtol=1e-12, atol=1e-12)
