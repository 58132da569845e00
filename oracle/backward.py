"""FP64 CPU oracle of the layer core's backward (first-order gradients).

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only ``tests/`` may use it;
the HIP library never does, and the two share no code.

The Megatron Core page "GDN Elementwise Fusion" (Execution and numerical
behavior) states that the fused stages support first-order autograd; the
Megatron-LM L2-fold pull request (Validation) and the flash-linear-attention
fused-conv pull request (Test plan) check input and parameter gradients.
Neither prints the backward formulas, so each function here is the plain
forward definition of a stage, written in float64 with PyTorch CPU tensors,
differentiated by autograd (a library primitive). Reading: the backward is the
derivative of the stage's exact function (the activation-dtype roundings of
the forward are treated as the identity), evaluated at the given stored
values.

The recurrence (``gated_delta_rule_fn``) is the gated delta rule written
token by token; its backward (``chunk_rule_bwd``) is autograd of it.

Parity status: pinned by finite differences (``torch.autograd.gradcheck``,
independent of autograd's own derivative rules) on small inputs and by closed
forms at special points (one token from a zero state, zero write strength,
the last write's value gradient); the recurrence's forward equals the pinned
C recurrence of ``gdn.py``. See ``tests/test_oracle_backward_pins.py``.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(x, grad=False):
    if x is None:
        return None
    t = torch.as_tensor(np.asarray(x, dtype=np.float64)).clone()
    return t.requires_grad_(grad)


def _np(t):
    return None if t is None else t.detach().numpy()


# --------------------------------------------------------------------------
# Gated RMSNorm: out = (o * r * w) * silu(gate), r = (mean(o^2) + eps)^-1/2
# --------------------------------------------------------------------------
def gated_rmsnorm_fn(o, gate, w, eps):
    """The forward of the gated norm (P2 option table, Execution and numerical
    behavior) on float64 tensors, without the activation-dtype roundings."""
    r = torch.rsqrt(torch.mean(o * o, dim=-1, keepdim=True) + eps)
    return (o * r * w) * (gate * torch.sigmoid(gate))


def gated_rmsnorm_bwd(o, gate, weight, dout, eps: float = 1e-5):
    """Gradients (d_o, d_gate, d_weight) of sum(dout * out). o, gate, dout:
    [..., dv]; weight: [dv]. d_weight sums over every row."""
    o_, g_, w_ = _t(o, True), _t(gate, True), _t(weight, True)
    out = gated_rmsnorm_fn(o_, g_, w_, eps)
    d = torch.autograd.grad(out, (o_, g_, w_), _t(dout))
    return tuple(_np(x) for x in d)


# --------------------------------------------------------------------------
# Prologue: conv + SiLU over q|k|v channels, beta and g
# --------------------------------------------------------------------------
def conv_silu_fn(x, w, bias, cu_seqlens=None):
    """Depthwise causal conv (tap j multiplies token t - 3 + j, zero history
    before each sequence start), bias, then SiLU (P3 Summary). x: [B, T, C];
    w: [C, K]; bias: [C] or None. With cu_seqlens, B is 1 and every packed
    sequence starts with zero history."""
    B, T, C = x.shape
    K = w.shape[1]

    def conv_one(xs):  # one sequence [L, C]
        L = xs.shape[0]
        acc = torch.zeros((L, C), dtype=x.dtype)
        if bias is not None:
            acc = acc + bias[None, :]
        for j in range(K):
            lag = K - 1 - j  # tap j reads token t - lag
            if lag >= L:
                continue
            shifted = torch.cat([torch.zeros((lag, C), dtype=x.dtype), xs[:L - lag]], 0)
            acc = acc + w[None, :, j] * shifted
        return acc

    if cu_seqlens is None:
        y = torch.stack([conv_one(x[i]) for i in range(B)], 0)
    else:
        cu = [int(c) for c in cu_seqlens]
        y = torch.cat([conv_one(x[0, cu[n]:cu[n + 1]]) for n in range(len(cu) - 1)], 0)[None]
    return y * torch.sigmoid(y)


def beta_g_fn(b, a, A_log, dt_bias):
    """beta = sigmoid(b); g = -exp(A_log) * softplus(a + dt_bias), softplus
    returning its argument above 20 (the forward's reading)."""
    beta = torch.sigmoid(b)
    sp = torch.nn.functional.softplus(a + dt_bias, beta=1.0, threshold=20.0)
    return beta, -torch.exp(A_log) * sp


def prologue_bwd(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, d_qkv, d_g, d_beta,
                 cu_seqlens=None):
    """Gradients of sum(d_qkv * qkv) + sum(d_g * g) + sum(d_beta * beta) with
    respect to x_q, x_k, x_v, conv_w, conv_b (None if absent), a, b, A_log and
    dt_bias. qkv is the concatenated conv output [B, T, C]."""
    xq, xk, xv = _t(x_q, True), _t(x_k, True), _t(x_v, True)
    w, bias = _t(conv_w, True), _t(conv_b, True)
    a_, b_, al, db_ = _t(a, True), _t(b, True), _t(A_log, True), _t(dt_bias, True)
    x = torch.cat([xq, xk, xv], -1)
    z = conv_silu_fn(x, w, bias, cu_seqlens)
    beta, g = beta_g_fn(b_, a_, al, db_)
    ins = [xq, xk, xv, w] + ([bias] if bias is not None else []) + [a_, b_, al, db_]
    d = torch.autograd.grad((z, g, beta), ins, (_t(d_qkv), _t(d_g), _t(d_beta)))
    d = [_np(t) for t in d]
    if bias is None:
        d.insert(4, None)
    return tuple(d)


# --------------------------------------------------------------------------
# The gated delta rule (the recurrence of gdn_chunk_rule_fwd)
# --------------------------------------------------------------------------
def _l2n(x, eps):
    return x / torch.sqrt(torch.sum(x * x, dim=-1, keepdim=True) + eps)


def gated_delta_rule_fn(q, k, v, g, beta, scale=1.0, use_qk_l2norm=True, l2_eps=1e-6,
                        cu_seqlens=None, initial_state=None):
    """The token-by-token recurrence on float64 tensors (Gated DeltaNet's
    gated delta rule, which the pages run in chunked form; P1 What/Why for the
    q/k normalisation folded into it):
        S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
        o_t = scale S_t q_t.
    q, k: [B, T, Hqk, dk]; v: [B, T, Hv, dv]; g, beta: [B, T, Hv]; value head
    h reads q/k head h // (Hv // Hqk). Returns (o [B, T, Hv, dv], final state
    [N, Hv, dv, dk])."""
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = Hv // Hqk
    if use_qk_l2norm:
        q, k = _l2n(q, l2_eps), _l2n(k, l2_eps)
    q = q.repeat_interleave(G, dim=2)
    k = k.repeat_interleave(G, dim=2)
    if cu_seqlens is None:
        spans = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(c) for c in cu_seqlens]
        spans = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    outs, finals = [], []
    for n, (b, t0, t1) in enumerate(spans):
        S = torch.zeros((Hv, dv, dk), dtype=q.dtype) if initial_state is None else initial_state[n]
        for t in range(t0, t1):
            kt, vt, qt = k[b, t], v[b, t], q[b, t]          # [Hv, dk], [Hv, dv], [Hv, dk]
            Sk = torch.einsum("hij,hj->hi", S, kt)
            S = torch.exp(g[b, t])[:, None, None] * (S - beta[b, t][:, None, None] * Sk[:, :, None] * kt[:, None, :]) \
                + beta[b, t][:, None, None] * vt[:, :, None] * kt[:, None, :]
            outs.append((b, t, scale * torch.einsum("hij,hj->hi", S, qt)))
        finals.append(S)
    rows = [[None] * T for _ in range(B)]
    for b, t, o in outs:
        rows[b][t] = o
    o = torch.stack([torch.stack(r, 0) if T else torch.zeros((0, Hv, dv), dtype=q.dtype) for r in rows], 0)
    return o, torch.stack(finals, 0)


def chunk_rule_bwd(q, k, v, g, beta, d_o, scale=1.0, use_qk_l2norm=True, l2_eps=1e-6,
                   cu_seqlens=None, initial_state=None, d_final_state=None):
    """Gradients (dq, dk, dv, dg, dbeta, d_initial_state) of
    sum(d_o * o) + sum(d_final_state * S_final) for gated_delta_rule_fn.
    d_initial_state is None when initial_state is None."""
    q_, k_, v_ = _t(q, True), _t(k, True), _t(v, True)
    g_, b_ = _t(g, True), _t(beta, True)
    h0 = _t(initial_state, True)
    o, fin = gated_delta_rule_fn(q_, k_, v_, g_, b_, scale, use_qk_l2norm, l2_eps, cu_seqlens, h0)
    outs, grads = [o], [_t(d_o)]
    if d_final_state is not None:
        outs.append(fin)
        grads.append(_t(d_final_state))
    ins = [q_, k_, v_, g_, b_] + ([h0] if h0 is not None else [])
    d = torch.autograd.grad(outs, ins, grads, allow_unused=True)
    d = [np.zeros(x.shape) if gr is None else _np(gr) for x, gr in zip(ins, d)]
    if h0 is None:
        d.append(None)
    return tuple(d)
