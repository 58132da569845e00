"""Pins of the backward oracle (oracle/backward.py) against things other than
autograd's own derivative rules: central finite differences
(torch.autograd.gradcheck) on small float64 inputs, and closed forms at
special points."""
import numpy as np
import pytest
import torch

from oracle import backward as OB
from oracle import gdn as O


def _r(rng, *shape):
    return torch.tensor(rng.normal(size=shape), dtype=torch.float64, requires_grad=True)


def test_gated_norm_gradients_match_finite_differences():
    rng = np.random.default_rng(1)
    o, gate, w = _r(rng, 3, 2, 8), _r(rng, 3, 2, 8), _r(rng, 8)
    assert torch.autograd.gradcheck(lambda o, g, w: OB.gated_rmsnorm_fn(o, g, w, 1e-5), (o, gate, w))


def test_gated_norm_forward_is_the_oracle_forward():
    rng = np.random.default_rng(2)
    o, gate, w = rng.normal(size=(4, 16)), rng.normal(size=(4, 16)), rng.normal(size=16)
    got = OB.gated_rmsnorm_fn(torch.tensor(o), torch.tensor(gate), torch.tensor(w), 1e-5).numpy()
    np.testing.assert_allclose(got, O.gated_rmsnorm(o, gate, w, 1e-5, "f64"), rtol=1e-13, atol=1e-15)


def test_gated_norm_gradient_closed_forms():
    rng = np.random.default_rng(3)
    o, w, dout = rng.normal(size=(5, 8)), rng.normal(size=8), rng.normal(size=(5, 8))
    # gate = 0: silu(0) = 0 and silu'(0) = 1/2, so d_o = d_w = 0 and
    # d_gate = dout * (o r w) / 2
    d_o, d_gate, d_w = OB.gated_rmsnorm_bwd(o, np.zeros((5, 8)), w, dout, 1e-5)
    r = 1 / np.sqrt(np.mean(o * o, -1, keepdims=True) + 1e-5)
    np.testing.assert_allclose(d_gate, dout * o * r * w / 2, rtol=1e-13)
    np.testing.assert_array_equal(d_o, 0.0)
    np.testing.assert_array_equal(d_w, 0.0)
    # scale invariance: out(c o) = out(o) for eps = 0, so <d_o, o> = 0 per row
    d_o, _, _ = OB.gated_rmsnorm_bwd(o, rng.normal(size=(5, 8)), w, dout, 0.0)
    np.testing.assert_allclose(np.sum(d_o * o, -1), 0.0, atol=1e-12)


def test_prologue_gradients_match_finite_differences():
    rng = np.random.default_rng(4)
    x, w, b = _r(rng, 2, 7, 3), _r(rng, 3, 4), _r(rng, 3)
    assert torch.autograd.gradcheck(lambda x, w, b: OB.conv_silu_fn(x, w, b), (x, w, b))
    xp = _r(rng, 1, 9, 3)
    cu = [0, 2, 2, 9]
    assert torch.autograd.gradcheck(lambda x, w: OB.conv_silu_fn(x, w, None, cu), (xp, w))
    bb, a, al, dtb = _r(rng, 2, 5, 3), _r(rng, 2, 5, 3), _r(rng, 3), _r(rng, 3)
    assert torch.autograd.gradcheck(lambda b, a, al, d: OB.beta_g_fn(b, a, al, d), (bb, a, al, dtb))


def test_prologue_forward_is_the_oracle_forward():
    rng = np.random.default_rng(5)
    x, w, bias = rng.normal(size=(2, 11, 6)), rng.uniform(-0.5, 0.5, (6, 4)), rng.normal(size=6)
    got = OB.conv_silu_fn(torch.tensor(x), torch.tensor(w), torch.tensor(bias)).numpy()
    np.testing.assert_allclose(got, O.causal_conv_silu(x, w, bias), rtol=1e-13, atol=1e-15)
    b, a, al, dtb = rng.normal(size=(2, 11, 3)), 30 * rng.normal(size=(2, 11, 3)), rng.normal(size=3), rng.normal(size=3)
    beta, g = OB.beta_g_fn(*(torch.tensor(v) for v in (b, a, al, dtb)))
    rb, rg = O.beta_and_g(b, a, al, dtb)
    np.testing.assert_allclose(beta.numpy(), rb, rtol=1e-14)
    np.testing.assert_allclose(g.numpy(), rg, rtol=1e-14)


def test_prologue_gradient_closed_forms():
    rng = np.random.default_rng(6)
    B, T, C1 = 1, 6, 2
    xq, xk, xv = (rng.normal(size=(B, T, C1)) for _ in range(3))
    C = 3 * C1
    w = np.zeros((C, 4))
    w[:, 3] = 1.0  # identity taps: qkv = silu(x)
    d_qkv = rng.normal(size=(B, T, C))
    Hv = 2
    a, b = np.zeros((B, T, Hv)), np.zeros((B, T, Hv))
    A_log, dt_bias = np.log([2.0, 3.0]), np.zeros(Hv)
    d_g, d_beta = rng.normal(size=(B, T, Hv)), rng.normal(size=(B, T, Hv))
    dxq, dxk, dxv, dw, dbias, da, db, dal, ddt = OB.prologue_bwd(
        xq, xk, xv, w, None, a, b, A_log, dt_bias, d_qkv, d_g, d_beta)
    x = np.concatenate([xq, xk, xv], -1)
    s = 1 / (1 + np.exp(-x))
    dsilu = s * (1 + x * (1 - s))
    np.testing.assert_allclose(np.concatenate([dxq, dxk, dxv], -1), d_qkv * dsilu, rtol=1e-13)
    # d_w[c, 3] = sum_t dy[t, c] x[t, c]; d_w[c, 2] = sum_t dy[t, c] x[t - 1, c]
    dy = d_qkv * dsilu
    np.testing.assert_allclose(dw[:, 3], np.sum(dy * x, (0, 1)), rtol=1e-12)
    np.testing.assert_allclose(dw[:, 2], np.sum(dy[:, 1:] * x[:, :-1], (0, 1)), rtol=1e-12)
    assert dbias is None
    # beta at b = 0: sigmoid' = 1/4; g at a + dt_bias = 0: softplus' = 1/2
    np.testing.assert_allclose(db, d_beta / 4, rtol=1e-14)
    np.testing.assert_allclose(da, -d_g * np.exp(A_log) / 2, rtol=1e-14)
    np.testing.assert_allclose(ddt, np.sum(-d_g * np.exp(A_log) / 2, (0, 1)), rtol=1e-13)
    np.testing.assert_allclose(dal, np.sum(-d_g * np.exp(A_log) * np.log(2.0), (0, 1)), rtol=1e-13)
