"""Pins of the oracle's backward pass (the reverse-mode derivative of the
recurrence of "Sostituire il motore", LT2 explainer, paithon.it, with the
read-out o_t = S_t^T q_t) for the loss  sum_t <dO_t, o_t> + <dS_L, S_L>.

Independent checks: torch autograd through a plain float64 torch loop over the
tokens (a library's derivative of the forward written here), central finite
differences of the oracle's own forward along random directions, the closed
form of the alpha = 1, beta = 0 case, and Euler's identity for the parts of the
map that are linear (o is linear in q; with S_0 = 0 the loss is linear in v;
with v = 0 it is linear in S_0).  A wrong sign, a missing erase or decay term,
a transposed state or an off-by-one token in the adjoint fails one of them.
Lengths above 64 exercise the oracle's segment checkpoints.
"""
import numpy as np
import pytest
import torch

import oracle


def case(seed, B, L, H, dk, dv, channel, lo=0.3):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, L, H, dk))
    k = g.standard_normal((B, L, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((B, L, H, dv))
    a = g.uniform(lo, 1.0, (B, L, H, dk) if channel else (B, L, H))
    b = g.uniform(0.0, 1.0, (B, L, H))
    S0 = g.standard_normal((B, H, dk, dv))
    dO = g.standard_normal((B, L, H, dv))
    dSL = g.standard_normal((B, H, dk, dv))
    return q, k, v, a, b, S0, dO, dSL


def torch_loss(q, k, v, la, b, S0, dO, dSL, channel):
    """Forward of the recurrence in torch (float64), returning the loss."""
    B, L, H, dk = q.shape
    loss = 0.0
    for bb in range(B):
        for h in range(H):
            S = S0[bb, h]
            for t in range(L):
                kt, vt, qt = k[bb, t, h], v[bb, t, h], q[bb, t, h]
                a = torch.exp(la[bb, t, h])
                P = S - b[bb, t, h] * torch.outer(kt, kt @ S)
                S = (a[:, None] if channel else a) * P + b[bb, t, h] * torch.outer(kt, vt)
                loss = loss + (S.T @ qt) @ dO[bb, t, h]
            loss = loss + (S * dSL[bb, h]).sum()
    return loss


@pytest.mark.parametrize("channel", [0, 1])
@pytest.mark.parametrize("L", [1, 9, 70])
def test_backward_matches_torch_autograd(channel, L):
    q, k, v, a, b, S0, dO, dSL = case(1 + L + channel, 2, L, 2, 4, 3, channel)
    ref = oracle.backward(q, k, v, a, b, dO, S0, dSL)
    T = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, np.log(a), b, S0)]
    loss = torch_loss(*T, torch.tensor(dO), torch.tensor(dSL), channel)
    loss.backward()
    for name, t in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"), T):
        np.testing.assert_allclose(ref[name], t.grad.numpy(), rtol=0, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("channel", [0, 1])
def test_backward_finite_differences(channel):
    q, k, v, a, b, S0, dO, dSL = case(7, 1, 12, 2, 5, 4, channel)
    g = oracle.backward(q, k, v, a, b, dO, S0, dSL)

    def loss(q, k, v, la, b, S0):
        o, S = oracle.prefill(q, k, v, np.exp(la), b, S0)
        return float((o * dO).sum() + (S * dSL).sum())

    base = [q, k, v, np.log(a), b, S0]
    names = ["dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"]
    rng = np.random.default_rng(8)
    eps = 1e-5
    for i, name in enumerate(names):
        d = rng.standard_normal(base[i].shape)
        plus = list(base)
        minus = list(base)
        plus[i] = base[i] + eps * d
        minus[i] = base[i] - eps * d
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        an = float((g[name] * d).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_backward_closed_form_alpha1_beta0():
    """alpha = 1, beta = 0: the state stays S_0, o_t = S_0^T q_t.  Then
    dq_t = S_0 dO_t, dv = 0, dk = 0, dlog_alpha_t = <G_t, S_0>, and
    dbeta_t = k^T G_t v_t - k^T G_t S_0^T k with G_t = dS_L + sum_{s>=t} q_s dO_s^T;
    dS_0 = G_1."""
    q, k, v, a, b, S0, dO, dSL = case(9, 1, 6, 1, 4, 3, 0)
    a[:] = 1.0
    b[:] = 0.0
    g = oracle.backward(q, k, v, a, b, dO, S0, dSL)
    S = S0[0, 0]
    G = dSL[0, 0].copy()
    for t in range(5, -1, -1):
        qt, kt, vt, dot = q[0, t, 0], k[0, t, 0], v[0, t, 0], dO[0, t, 0]
        G = G + np.outer(qt, dot)
        np.testing.assert_allclose(g["dq"][0, t, 0], S @ dot, atol=1e-13)
        np.testing.assert_allclose(g["dlog_alpha"][0, t, 0], (G * S).sum(), atol=1e-12)
        np.testing.assert_allclose(g["dbeta"][0, t, 0], kt @ G @ vt - kt @ G @ (S.T @ kt), atol=1e-12)
    assert np.all(g["dv"] == 0.0) and np.all(g["dk"] == 0.0)
    np.testing.assert_allclose(g["dS0"][0, 0], G, atol=1e-13)


@pytest.mark.parametrize("channel", [0, 1])
def test_backward_euler_identities(channel):
    q, k, v, a, b, S0, dO, dSL = case(10, 2, 20, 2, 4, 5, channel)
    # o is linear in q (with dS_L = 0): <dq, q> = <dO, o>
    o, _ = oracle.prefill(q, k, v, a, b, S0)
    g = oracle.backward(q, k, v, a, b, dO, S0, None)
    np.testing.assert_allclose((g["dq"] * q).sum(), (dO * o).sum(), rtol=1e-12)
    # with S_0 = 0 the loss is linear in v
    o, S = oracle.prefill(q, k, v, a, b, None)
    g = oracle.backward(q, k, v, a, b, dO, None, dSL)
    np.testing.assert_allclose((g["dv"] * v).sum(), (dO * o).sum() + (dSL * S).sum(), rtol=1e-12)
    # with v = 0 the loss is linear in S_0
    z = np.zeros_like(v)
    o, S = oracle.prefill(q, k, z, a, b, S0)
    g = oracle.backward(q, k, z, a, b, dO, S0, dSL)
    np.testing.assert_allclose((g["dS0"] * S0).sum(), (dO * o).sum() + (dSL * S).sum(), rtol=1e-12)
