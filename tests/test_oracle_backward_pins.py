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


# --------------------------------------------------------------------------
# The gated delta rule's backward
# --------------------------------------------------------------------------
def _rule_inputs(rng, B, T, Hqk, dk, Hv, dv):
    return (rng.normal(size=(B, T, Hqk, dk)), rng.normal(size=(B, T, Hqk, dk)), rng.normal(size=(B, T, Hv, dv)),
            -rng.uniform(0.01, 1.0, (B, T, Hv)), rng.uniform(0.05, 1.0, (B, T, Hv)))


@pytest.mark.parametrize("use_l2,cu", [(True, None), (False, None), (True, [0, 3, 3, 10])])
def test_rule_forward_is_the_oracle_forward(use_l2, cu):
    rng = np.random.default_rng(10)
    B = 1 if cu else 2
    q, k, v, g, b = _rule_inputs(rng, B, 10, 2, 8, 4, 6)
    N = len(cu) - 1 if cu else B
    h0 = rng.normal(size=(N, 4, 6, 8))
    o, fin = OB.gated_delta_rule_fn(*(torch.tensor(x) for x in (q, k, v, g, b)), 0.7, use_l2, 1e-6, cu,
                                    torch.tensor(h0))
    ro, rfin = O.gated_delta_rule(q, k, v, g, b, 0.7, use_l2, 1e-6, cu, h0, True)
    np.testing.assert_allclose(o.numpy(), ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fin.numpy(), rfin, rtol=1e-12, atol=1e-13)


def test_rule_gradients_match_finite_differences():
    rng = np.random.default_rng(11)
    q, k, v, g, b = (torch.tensor(x, requires_grad=True) for x in _rule_inputs(rng, 1, 6, 1, 3, 2, 2))
    h0 = torch.tensor(rng.normal(size=(2, 2, 2, 3)), requires_grad=True)
    cu = [0, 4, 6]

    def f(q, k, v, g, b, h0):
        o, fin = OB.gated_delta_rule_fn(q, k, v, g, b, 0.6, True, 1e-6, cu, h0)
        return o, fin

    assert torch.autograd.gradcheck(f, (q, k, v, g, b, h0))


def test_rule_gradient_closed_form_one_token_from_zero():
    # S = beta v k^T and o = scale beta (k.q) v with unit q, k: dv = scale beta
    # (k.q) dO, dbeta = scale (k.q) (v.dO), dg = 0 (the decay multiplies S0 = 0)
    rng = np.random.default_rng(12)
    q, k, v, g, b = _rule_inputs(rng, 1, 1, 1, 5, 1, 4)
    dO = rng.normal(size=(1, 1, 1, 4))
    dq, dk, dv, dg, db, dh0 = OB.chunk_rule_bwd(q, k, v, g, b, dO, 0.8)
    qh, kh = O.l2norm(q), O.l2norm(k)
    kq = float(np.sum(qh * kh))
    np.testing.assert_allclose(dv, 0.8 * b[..., None] * kq * dO, rtol=1e-12)
    np.testing.assert_allclose(db, 0.8 * kq * np.sum(v * dO, -1), rtol=1e-12)
    np.testing.assert_array_equal(dg, 0.0)
    assert dh0 is None
    # d/dq of (qh . c) with qh = q / |q| (eps 1e-6) is (c - qh (qh . c)) / |q|
    c = 0.8 * b[0, 0, 0] * kh[0, 0, 0] * float(np.sum(v * dO))
    n = np.sqrt(np.sum(q * q) + 1e-6)
    np.testing.assert_allclose(dq[0, 0, 0], (c - qh[0, 0, 0] * np.dot(qh[0, 0, 0], c)) / n, rtol=1e-10)


def test_rule_gradient_closed_form_zero_write_strength():
    # beta = 0: S_t = exp(G_t) S0 with G_t the running sum of g, so
    # o_t = scale exp(G_t) S0 q_t, dv = 0, dS0 = scale sum_t exp(G_t) dO_t q_t^T
    # and dg_t = sum_{u >= t} scale exp(G_u) dO_u . (S0 q_u)
    rng = np.random.default_rng(13)
    q, k, v, g, _ = _rule_inputs(rng, 1, 5, 1, 4, 1, 3)
    b = np.zeros((1, 5, 1))
    h0 = rng.normal(size=(1, 1, 3, 4))
    dO = rng.normal(size=(1, 5, 1, 3))
    dq, dk, dv, dg, db, dh0 = OB.chunk_rule_bwd(q, k, v, g, b, dO, 0.5, False, 0.0, None, h0)
    G = np.cumsum(g[0, :, 0])
    qs = q[0, :, 0]
    np.testing.assert_array_equal(dv, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_allclose(dh0[0, 0], 0.5 * np.einsum("t,ti,tj->ij", np.exp(G), dO[0, :, 0], qs), rtol=1e-12)
    per = 0.5 * np.exp(G) * np.einsum("ti,ij,tj->t", dO[0, :, 0], h0[0, 0], qs)
    np.testing.assert_allclose(dg[0, :, 0], np.cumsum(per[::-1])[::-1], rtol=1e-12)
    np.testing.assert_allclose(dq[0, :, 0], 0.5 * np.exp(G)[:, None] * (dO[0, :, 0] @ h0[0, 0]), rtol=1e-12)


def test_rule_gradient_of_the_final_state_alone():
    # With dO = 0 and dS_T = I-like probe E_ij, the gradient of v_T (last token)
    # is beta_T E k_T (the last write is beta_T v_T k_T^T, nothing decays it)
    rng = np.random.default_rng(14)
    q, k, v, g, b = _rule_inputs(rng, 1, 4, 1, 3, 1, 2)
    dO = np.zeros((1, 4, 1, 2))
    E = rng.normal(size=(1, 1, 2, 3))
    _, _, dv, _, _, _ = OB.chunk_rule_bwd(q, k, v, g, b, dO, 1.0, True, 1e-6, None, None, E)
    kh = O.l2norm(k)
    np.testing.assert_allclose(dv[0, 3, 0], b[0, 3, 0] * E[0, 0] @ kh[0, 3, 0], rtol=1e-12)
