"""Pins of the FP64 oracle against facts the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a closed form, a
library routine, exact rational arithmetic, an independent formulation (matrix
products of transition maps, the chunked WY form) or an invariant the pages
state (P1 = Megatron-LM "fold q/k L2-norm into the gated_delta_rule kernel",
P2 = Megatron Core "GDN Elementwise Fusion", P3 = flash-linear-attention
"fused q/k/v short conv").
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from linear_attention_rnn_qkv_amd import synth
from oracle import gdn as O
from oracle.chunked import chunked_gated_delta_rule

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------------------
# round_to
# ----------------------------------------------------------------------------
def test_round_to_f16_matches_numpy():
    x = np.concatenate([RNG.standard_normal(5000) * 10.0 ** RNG.integers(-9, 5, 5000),
                        [0.0, -0.0, 65504.0, 65520.0, 1e-8, 6e-8, 2.0 ** -25]])
    np.testing.assert_array_equal(O.round_to(x, "f16"), x.astype(np.float16).astype(np.float64))


def test_round_to_bf16_matches_torch_on_float32_values():
    x = (RNG.standard_normal(20000) * 10.0 ** RNG.integers(-30, 30, 20000)).astype(np.float32)
    x = np.concatenate([x, np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, 2.0 ** -130, 3e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to(x.astype(np.float64), "bf16"), ref)


def test_round_to_bf16_ties_to_even():
    assert O.round_to(np.array([1 + 2 ** -8]), "bf16")[0] == 1.0
    assert O.round_to(np.array([1 + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6


def test_round_to_f32_matches_numpy():
    x = RNG.standard_normal(5000) * 10.0 ** RNG.integers(-40, 38, 5000)
    np.testing.assert_array_equal(O.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


# ----------------------------------------------------------------------------
# Concatenated depthwise causal conv + SiLU (P3 Summary / Why)
# ----------------------------------------------------------------------------
def _torch_conv_silu(x, w, bias=None):
    """Library route: conv1d with groups=C, left padding K-1, then SiLU."""
    B, T, C = x.shape
    K = w.shape[1]
    xt = torch.from_numpy(x).permute(0, 2, 1)
    wt = torch.from_numpy(w).unsqueeze(1)
    bt = None if bias is None else torch.from_numpy(bias)
    y = F.conv1d(F.pad(xt, (K - 1, 0)), wt, bt, groups=C)
    return F.silu(y).permute(0, 2, 1).numpy()


def test_conv_matches_library_conv1d():
    x = RNG.standard_normal((2, 37, 24))
    w = RNG.uniform(-0.5, 0.5, (24, 4))
    b = RNG.standard_normal(24)
    np.testing.assert_allclose(O.causal_conv_silu(x, w), _torch_conv_silu(x, w), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(O.causal_conv_silu(x, w, b), _torch_conv_silu(x, w, b), rtol=1e-13, atol=1e-14)


def test_concatenated_conv_equals_three_separate_convs_exactly():
    # P3 (Why, Test plan): one wide depthwise conv equals the three separate ones.
    xq, xk, xv = (RNG.standard_normal((1, 50, n)) for n in (8, 8, 16))
    wq, wk, wv = (RNG.uniform(-0.5, 0.5, (n, 4)) for n in (8, 8, 16))
    cat = O.causal_conv_silu(np.concatenate([xq, xk, xv], -1), np.concatenate([wq, wk, wv], 0))
    sep = np.concatenate([O.causal_conv_silu(xq, wq), O.causal_conv_silu(xk, wk),
                          O.causal_conv_silu(xv, wv)], -1)
    np.testing.assert_array_equal(cat, sep)


def test_identity_taps_give_silu():
    x = RNG.standard_normal((1, 20, 6))
    w = np.zeros((6, 4)); w[:, 3] = 1.0
    np.testing.assert_allclose(O.causal_conv_silu(x, w), F.silu(torch.from_numpy(x)).numpy(),
                               rtol=1e-15, atol=0)
    b = RNG.standard_normal(6)
    y = O.causal_conv_silu(x, np.zeros((6, 4)), b)
    np.testing.assert_allclose(y, np.broadcast_to(F.silu(torch.from_numpy(b)).numpy(), y.shape), rtol=1e-15)


def test_conv_is_causal():
    x = RNG.standard_normal((1, 30, 5))
    w = RNG.uniform(-0.5, 0.5, (5, 4))
    y0 = O.causal_conv_silu(x, w)
    x2 = x.copy(); x2[0, 17:] += 3.0
    y1 = O.causal_conv_silu(x2, w)
    np.testing.assert_array_equal(y0[0, :17], y1[0, :17])
    assert np.all(y0[0, 17] != y1[0, 17])


def test_conv_varlen_restarts_history():
    lens = [5, 1, 9, 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = RNG.standard_normal((1, cu[-1], 7))
    w = RNG.uniform(-0.5, 0.5, (7, 4))
    y = O.causal_conv_silu(x, w, cu_seqlens=cu)
    for n in range(len(lens)):
        np.testing.assert_array_equal(y[:, cu[n]:cu[n + 1]], O.causal_conv_silu(x[:, cu[n]:cu[n + 1]], w))


# ----------------------------------------------------------------------------
# beta and g (P2 option table: beta and decay preparation)
# ----------------------------------------------------------------------------
def test_beta_g_special_values():
    beta, g = O.beta_and_g(np.array([0.0, math.log(3.0), -math.log(3.0)]),
                           np.array([0.0, 0.0, 0.0]), np.array([math.log(2.0)] * 3),
                           np.array([0.0] * 3))
    np.testing.assert_allclose(beta, [0.5, 0.75, 0.25], rtol=1e-15)
    np.testing.assert_allclose(g, [-2.0 * math.log(2.0)] * 3, rtol=1e-15)  # softplus(0) = ln 2
    _, g1 = O.beta_and_g(np.zeros(1), np.array([math.log(math.e - 1.0) - 0.25]),
                         np.array([1.5]), np.array([0.25]))
    np.testing.assert_allclose(g1, [-math.exp(1.5)], rtol=1e-14)  # softplus = 1


def test_beta_g_match_library_functions():
    b = RNG.standard_normal(1000) * 4
    a = RNG.standard_normal(1000) * 4
    A_log = np.log(RNG.uniform(1, 16, 1000))
    dtb = RNG.normal(0, 0.1, 1000)
    beta, g = O.beta_and_g(b, a, A_log, dtb)
    np.testing.assert_allclose(beta, torch.sigmoid(torch.from_numpy(b)).numpy(), rtol=1e-14)
    np.testing.assert_allclose(g, -np.exp(A_log) * np.logaddexp(0.0, a + dtb), rtol=1e-13)
    assert np.all((beta > 0) & (beta < 1)) and np.all(g < 0) and np.all(np.exp(g) < 1)


# ----------------------------------------------------------------------------
# L2 norm (P1 Why: eps 1e-6, per head over the last dim)
# ----------------------------------------------------------------------------
def test_l2norm_identity():
    x = RNG.standard_normal((3, 7, 64)) * 10.0 ** RNG.integers(-4, 2, (3, 7, 1))
    y = O.l2norm(x, 1e-6)
    s = np.sum(x * x, -1)
    np.testing.assert_allclose(np.sum(y * y, -1), s / (s + 1e-6), rtol=1e-13)
    cos = np.sum(x * y, -1) / np.linalg.norm(x, axis=-1) / np.linalg.norm(y, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)
    np.testing.assert_allclose(O.l2norm(x, 0.0), x / np.linalg.norm(x, axis=-1, keepdims=True), rtol=1e-14)


# ----------------------------------------------------------------------------
# The recurrence
# ----------------------------------------------------------------------------
def _rand_problem(B=1, T=9, Hqk=1, dk=4, Hv=1, dv=3, seed=0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, Hqk, dk))
    k = r.standard_normal((B, T, Hqk, dk))
    v = r.standard_normal((B, T, Hv, dv))
    g = -r.uniform(0.0, 1.0, (B, T, Hv))
    beta = r.uniform(0.0, 1.0, (B, T, Hv))
    return q, k, v, g, beta


def test_single_token_closed_form():
    q, k, v, g, beta = _rand_problem(T=1, dk=5, dv=3)
    o, _ = O.gated_delta_rule(q, k, v, g, beta, scale=0.7)
    qn, kn = O.l2norm(q), O.l2norm(k)
    expect = 0.7 * beta[0, 0, 0] * np.dot(kn[0, 0, 0], qn[0, 0, 0]) * v[0, 0, 0]
    np.testing.assert_allclose(o[0, 0, 0], expect, rtol=1e-14)


def test_scalar_recurrence_geometric_series():
    # dk = dv = 1, unit key and query, constant g, beta, v:
    # S_t = e^g (1 - beta) S_{t-1} + beta v  =>  S_t = beta v (1 - rho^t) / (1 - rho)
    T, gval, bval, vval = 40, -0.3, 0.6, 1.7
    rho = math.exp(gval) * (1.0 - bval)
    ones = np.ones((1, T, 1, 1))
    o, fin = O.gated_delta_rule(ones, ones, vval * ones, np.full((1, T, 1), gval),
                                np.full((1, T, 1), bval), use_qk_l2norm=False,
                                output_final_state=True)
    t = np.arange(1, T + 1)
    np.testing.assert_allclose(o[0, :, 0, 0], bval * vval * (1 - rho ** t) / (1 - rho), rtol=1e-13)
    np.testing.assert_allclose(fin[0, 0, 0, 0], bval * vval * (1 - rho ** T) / (1 - rho), rtol=1e-13)


def _brute_state(kn, v, g, beta, upto):
    """S_t = sum_s beta_s v_s k_s^T prod_{r=s+1..t} e^{g_r} (I - beta_r k_r k_r^T)."""
    dk, dv = kn.shape[1], v.shape[1]
    S = np.zeros((dv, dk))
    for s in range(upto):
        M = np.eye(dk)
        for r in range(s + 1, upto):
            M = M @ (math.exp(g[r]) * (np.eye(dk) - beta[r] * np.outer(kn[r], kn[r])))
        S += beta[s] * np.outer(v[s], kn[s]) @ M
    return S


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_brute_force_transition_products(T):
    q, k, v, g, beta = _rand_problem(T=T, dk=4, dv=3, seed=T)
    o, fin = O.gated_delta_rule(q, k, v, g, beta, scale=0.5, output_final_state=True)
    qn, kn = O.l2norm(q)[0, :, 0], O.l2norm(k)[0, :, 0]
    for t in range(T):
        S = _brute_state(kn, v[0, :, 0], g[0, :, 0], beta[0, :, 0], t + 1)
        np.testing.assert_allclose(o[0, t, 0], 0.5 * S @ qn[t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], _brute_state(kn, v[0, :, 0], g[0, :, 0], beta[0, :, 0], T),
                               rtol=1e-12, atol=1e-14)


def test_exact_rational_arithmetic():
    # Exact arithmetic on the same (binary) inputs: the FP64 result must agree
    # to a few ulps. Uses the factored form S (I - b k k^T) literally.
    q, k, v, g, beta = _rand_problem(T=4, dk=2, dv=3, seed=7)
    o, _ = O.gated_delta_rule(q, k, v, g, beta, use_qk_l2norm=False)
    Fr = Fraction
    S = [[Fr(0)] * 2 for _ in range(3)]
    for t in range(4):
        kk = [Fr(x) for x in k[0, t, 0]]
        qq = [Fr(x) for x in q[0, t, 0]]
        d, b = Fr(math.exp(g[0, t, 0])), Fr(beta[0, t, 0])
        M = [[(1 if i == j else 0) - b * kk[i] * kk[j] for j in range(2)] for i in range(2)]
        S = [[d * sum(S[r][m] * M[m][c] for m in range(2)) + b * Fr(v[0, t, 0, r]) * kk[c]
              for c in range(2)] for r in range(3)]
        exact = [float(sum(S[r][c] * qq[c] for c in range(2))) for r in range(3)]
        np.testing.assert_allclose(o[0, t, 0], exact, rtol=1e-13, atol=1e-15)


def test_orthonormal_keys_retrieve_values_exactly():
    # g = 0, beta = 1 and orthonormal keys: writing (k_j, v_j) makes S k_j = v_j,
    # so querying q = k_j later (beta = 0, no write) returns scale * v_j.
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(RNG.standard_normal((dk, dk)))
    keys = Qm[:, :n].T
    vals = RNG.standard_normal((n, dv))
    T = 2 * n
    k = np.zeros((1, T, 1, dk)); k[0, :n, 0] = keys; k[0, n:, 0] = keys
    q = np.zeros((1, T, 1, dk)); q[0, :n, 0] = keys; q[0, n:, 0] = keys[::-1]
    v = np.zeros((1, T, 1, dv)); v[0, :n, 0] = vals
    beta = np.zeros((1, T, 1)); beta[0, :n] = 1.0
    o, _ = O.gated_delta_rule(q, k, v, np.zeros((1, T, 1)), beta, scale=2.0, use_qk_l2norm=False)
    np.testing.assert_allclose(o[0, :n, 0], 2.0 * vals, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o[0, n:, 0], 2.0 * vals[::-1], rtol=1e-12, atol=1e-12)


def test_unit_key_write_is_read_back_for_any_keys():
    # beta = 1 with unit keys: S_t k_t = v_t even when keys are not orthogonal.
    q, k, v, g, _ = _rand_problem(T=12, dk=6, dv=4, seed=3)
    kn = O.l2norm(k, 0.0)
    o, _ = O.gated_delta_rule(kn, kn, v, g, np.ones_like(g), use_qk_l2norm=False)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


def test_beta_zero_only_decays_initial_state():
    q, k, v, g, _ = _rand_problem(T=10, dk=4, dv=3, seed=5)
    S0 = RNG.standard_normal((1, 1, 3, 4))
    o, fin = O.gated_delta_rule(q, k, v, g, np.zeros_like(g), scale=1.3, initial_state=S0,
                                output_final_state=True)
    qn = O.l2norm(q)
    cg = np.cumsum(g[0, :, 0])
    for t in range(10):
        np.testing.assert_allclose(o[0, t, 0], 1.3 * math.exp(cg[t]) * S0[0, 0] @ qn[0, t, 0], rtol=1e-13)
    np.testing.assert_allclose(fin[0, 0], math.exp(cg[-1]) * S0[0, 0], rtol=1e-13)


def test_flag_off_is_a_no_op_and_in_kernel_equals_caller_side():
    # P1 (Why): use_qk_l2norm=False is a no-op; in-kernel and caller-side
    # normalisation use the same eps and give the same result.
    q, k, v, g, beta = _rand_problem(T=20, dk=8, dv=4, seed=11)
    o_in, _ = O.gated_delta_rule(q, k, v, g, beta, use_qk_l2norm=True)
    o_caller, _ = O.gated_delta_rule(O.l2norm(q), O.l2norm(k), v, g, beta, use_qk_l2norm=False)
    np.testing.assert_array_equal(o_in, o_caller)


def test_gqa_map_equals_explicit_replication():
    # P1 (Why): per-head normalisation makes head replication result-neutral.
    q, k, v, g, beta = _rand_problem(T=15, Hqk=2, dk=4, Hv=6, dv=3, seed=2)
    o, _ = O.gated_delta_rule(q, k, v, g, beta)
    rep = np.repeat(np.arange(2), 3)  # value head h reads key head h // 3
    o2, _ = O.gated_delta_rule(q[:, :, rep], k[:, :, rep], v, g, beta)
    np.testing.assert_array_equal(o, o2)
    o3, _ = O.gated_delta_rule(O.l2norm(q)[:, :, rep], O.l2norm(k)[:, :, rep], v, g, beta,
                               use_qk_l2norm=False)
    np.testing.assert_array_equal(o, o3)


@pytest.mark.parametrize("chunk", [1, 7, 64, 200])
def test_chunked_form_equals_sequential(chunk):
    q, k, v, g, beta = _rand_problem(B=2, T=150, Hqk=1, dk=16, Hv=2, dv=8, seed=chunk)
    g = g * 0.2  # keep state alive across chunk boundaries
    S0 = RNG.standard_normal((2, 2, 8, 16))
    o, fin = O.gated_delta_rule(q, k, v, g, beta, scale=0.25, initial_state=S0, output_final_state=True)
    oc, finc = chunked_gated_delta_rule(q, k, v, g, beta, scale=0.25, chunk=chunk, initial_state=S0)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(finc, fin, rtol=1e-10, atol=1e-12)


def test_varlen_equals_separate_runs():
    lens = [7, 1, 20, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = _rand_problem(T=cu[-1], Hqk=1, dk=4, Hv=2, dv=3, seed=9)
    S0 = RNG.standard_normal((4, 2, 3, 4))
    o, fin = O.gated_delta_rule(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0, output_final_state=True)
    for n in range(4):
        s = slice(cu[n], cu[n + 1])
        o1, f1 = O.gated_delta_rule(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s],
                                    initial_state=S0[n:n + 1], output_final_state=True)
        np.testing.assert_array_equal(o[:, s], o1)
        np.testing.assert_array_equal(fin[n], f1[0])


def test_state_handoff_equals_one_run():
    q, k, v, g, beta = _rand_problem(T=30, dk=4, dv=3, seed=4)
    o, fin = O.gated_delta_rule(q, k, v, g, beta, output_final_state=True)
    oa, fa = O.gated_delta_rule(q[:, :13], k[:, :13], v[:, :13], g[:, :13], beta[:, :13],
                                output_final_state=True)
    ob, fb = O.gated_delta_rule(q[:, 13:], k[:, 13:], v[:, 13:], g[:, 13:], beta[:, 13:],
                                initial_state=fa, output_final_state=True)
    np.testing.assert_array_equal(np.concatenate([oa, ob], 1), o)
    np.testing.assert_array_equal(fb, fin)


def test_work_split_does_not_change_results():
    q, k, v, g, beta = _rand_problem(B=2, T=40, Hqk=2, dk=8, Hv=4, dv=20, seed=8)
    ref, _ = O.gated_delta_rule(q, k, v, g, beta, threads=1, rows_per_unit=20)
    for rpu, th in [(1, 3), (16, 4), (7, 2)]:
        o, _ = O.gated_delta_rule(q, k, v, g, beta, threads=th, rows_per_unit=rpu)
        np.testing.assert_array_equal(o, ref)


# ----------------------------------------------------------------------------
# Output RMSNorm + SiLU gate (P2 option table; Execution and numerical behavior)
# ----------------------------------------------------------------------------
def test_gated_norm_matches_library_rms_norm_and_silu():
    o = RNG.standard_normal((3, 5, 2, 64))
    gate = RNG.standard_normal((3, 5, 2, 64))
    w = 1 + RNG.normal(0, 0.02, 64)
    ref_y = F.rms_norm(torch.from_numpy(o), (64,), torch.from_numpy(w), eps=1e-5).numpy()
    for act in ("f32", "bf16", "f16"):
        y = O.round_to(ref_y, act)
        ref = O.round_to(y * F.silu(torch.from_numpy(gate)).numpy(), act)
        got = O.gated_rmsnorm(o, gate, w, 1e-5, act)
        # equal except where the float64 product sits within an ulp of a tie
        np.testing.assert_allclose(got, ref, rtol=2.0 ** -(8 if act == "bf16" else 11), atol=0)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_gated_norm_materialises_the_norm_in_the_activation_dtype(act):
    """Reading R6 (the norm result is rounded to the activation dtype before
    the FP32 gate multiply), pinned exactly. The expected values come from
    library routines: torch's float64 rms_norm, torch's conversion to the
    16-bit dtype, torch's silu. Inputs are 16-bit values; the weight is
    drawn as 16-bit values too. The gate is chosen so that silu(gate) is
    not a power of two, so rounding the norm result first changes the final
    rounded output for many elements: an oracle that skipped that rounding
    (or rounded the gate product only) fails the exact comparison."""
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[act]
    rng = np.random.default_rng(606)
    o = torch.from_numpy(rng.standard_normal((64, 128))).to(dt).double()
    w = torch.from_numpy(1 + rng.normal(0, 0.02, 128)).to(dt).double()
    gate = torch.from_numpy(rng.standard_normal((64, 128)) * 3).to(dt).double()
    y = F.rms_norm(o, (128,), w, eps=1e-5).to(dt).double()       # materialised norm
    ref = (y * F.silu(gate)).to(dt).double().numpy()
    got = O.gated_rmsnorm(o.numpy(), gate.numpy(), w.numpy(), 1e-5, act)
    np.testing.assert_array_equal(got, ref)
    # the pin has power: without the intermediate rounding the outputs differ
    skip = (F.rms_norm(o, (128,), w, eps=1e-5) * F.silu(gate)).to(dt).double().numpy()
    assert np.mean(skip != ref) > 0.05


def test_gated_norm_rms_identity_gate_zero_and_scale_invariance():
    o = RNG.standard_normal((4, 3, 32)) * 10.0 ** RNG.integers(-2, 2, (4, 3, 1))
    w = 1 + RNG.normal(0, 0.02, 32)
    big = np.full_like(o, 40.0)  # silu(40) == 40 to float64 precision
    y = O.gated_rmsnorm(o, big, w, 1e-5, "f64") / 40.0
    m = np.mean(o * o, -1)
    np.testing.assert_allclose(np.sqrt(np.mean((y / w) ** 2, -1)), np.sqrt(m / (m + 1e-5)), rtol=1e-12)
    assert np.all(O.gated_rmsnorm(o, np.zeros_like(o), w, 1e-5, "bf16") == 0)
    gate = RNG.standard_normal(o.shape)
    a = O.gated_rmsnorm(o, gate, w, 0.0, "f64")
    b = O.gated_rmsnorm(3.7 * o, gate, w, 0.0, "f64")
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------
# The layer composition
# ----------------------------------------------------------------------------
def test_layer_concatenated_prologue_equals_separate_route():
    from linear_attention_rnn_qkv_amd import synth
    s = synth.spec(0).replace(T=40)
    x = synth.make_inputs(s)
    f = synth.to_f64
    kw = dict(Hqk=s.Hqk, dk=s.dk, Hv=s.Hv, dv=s.dv, act=s.act, scale=s.dk ** -0.5)
    out, st = O.layer(f(x["x_q"]), f(x["x_k"]), f(x["x_v"]), f(x["conv_w"]), None, f(x["a"]),
                      f(x["b"]), f(x["A_log"]), f(x["dt_bias"]), f(x["gate"]), f(x["norm_w"]),
                      return_stages=True, **kw)
    nq = s.Hqk * s.dk
    w = f(x["conv_w"])
    sep = [O.round_to(O.causal_conv_silu(f(x[n]), w[a:b]), s.act)
           for n, a, b in (("x_q", 0, nq), ("x_k", nq, 2 * nq), ("x_v", 2 * nq, s.C))]
    np.testing.assert_array_equal(st["qkv"], np.concatenate(sep, -1))
    assert np.all(np.isfinite(out)) and out.shape == (1, 40, s.Hv, s.dv)


# ----------------------------------------------------------------------------
# Recurrent decode
# ----------------------------------------------------------------------------
def _decode_run(x, s, T, scale):
    """T decode steps from a zero cache and state over the tokens of x."""
    f = synth.to_f64
    B = s.B
    cache = np.zeros((B, 3, s.C))
    S = np.zeros((B, s.Hv, s.dv, s.dk))
    outs, caches = [], []
    for t in range(T):
        o, cache, S = O.decode_step(
            f(x["x_q"])[:, t], f(x["x_k"])[:, t], f(x["x_v"])[:, t], f(x["conv_w"]), None, cache,
            f(x["a"])[:, t], f(x["b"])[:, t], f(x["A_log"]), f(x["dt_bias"]), S, f(x["gate"])[:, t],
            f(x["norm_w"]), Hqk=s.Hqk, dk=s.dk, Hv=s.Hv, dv=s.dv, act=s.act, scale=scale)
        outs.append(o)
        caches.append(cache)
    return np.stack(outs, 1), caches, S


def test_decode_steps_from_zero_equal_the_layer():
    # The recurrent form and the sequence form of the same layer: token t of
    # the layer's output equals the t-th decode step; the final state equals
    # the recurrence's final state (conv lags, tap order, gates, GQA map and
    # every rounding point are exercised by the comparison).
    s = synth.spec(0).replace(B=2, T=11, Hqk=2, dk=8, Hv=4, dv=6, act="bf16", gate_dtype="bf16",
                              w_dtype="bf16")
    x = synth.make_inputs(s)
    f = synth.to_f64
    scale = 0.3
    got, caches, S = _decode_run(x, s, s.T, scale)
    ref, st = O.layer(f(x["x_q"]), f(x["x_k"]), f(x["x_v"]), f(x["conv_w"]), None, f(x["a"]),
                      f(x["b"]), f(x["A_log"]), f(x["dt_bias"]), f(x["gate"]), f(x["norm_w"]),
                      Hqk=s.Hqk, dk=s.dk, Hv=s.Hv, dv=s.dv, act=s.act, scale=scale,
                      return_stages=True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    q, k, v = (a.reshape(s.B, s.T, -1, d) for a, d in
               ((st["qkv"][..., :16], s.dk), (st["qkv"][..., 16:32], s.dk), (st["qkv"][..., 32:], s.dv)))
    _, fin = O.gated_delta_rule(q, k, v, st["g"], st["beta"], scale=scale, output_final_state=True)
    np.testing.assert_allclose(S, fin, rtol=1e-10, atol=1e-12)
    # the cache after step t holds inputs t-2, t-1, t exactly (zeros before the start)
    xc = np.concatenate([f(x["x_q"]), f(x["x_k"]), f(x["x_v"])], -1)
    pad = np.concatenate([np.zeros((s.B, 2, s.C)), xc], 1)
    for t in (0, 1, 5, s.T - 1):
        np.testing.assert_array_equal(caches[t], pad[:, t:t + 3])


def test_decode_unit_write_strength_overwrites_the_value_at_the_key():
    # With beta = 1 and no decay the delta rule replaces what the state held
    # at the (unit) key by the new value, whatever the state was: S_new k = v.
    rng = np.random.default_rng(5)
    Hqk, dk, Hv, dv = 1, 8, 2, 5
    C = 2 * Hqk * dk + Hv * dv
    xq, xk, xv = rng.normal(size=(1, dk)), rng.normal(size=(1, dk)), rng.normal(size=(1, Hv * dv))
    w = rng.uniform(-0.5, 0.5, (C, 4))
    cache = rng.normal(size=(1, 3, C))
    S0 = rng.normal(size=(1, Hv, dv, dk))
    b = np.full((1, Hv), 60.0)           # sigmoid(60) == 1 in float64
    a = np.zeros((1, Hv))
    A_log = np.full(Hv, -80.0)           # exp(-80) softplus(0): decay e^g == 1 in float64
    out, _, S = O.decode_step(xq, xk, xv, w, None, cache, a, b, A_log, np.zeros(Hv), S0,
                              np.zeros((1, Hv, dv)), np.ones(dv), Hqk=Hqk, dk=dk, Hv=Hv, dv=dv,
                              act="f64", scale=1.0, l2_eps=0.0)
    win = np.concatenate([cache[0], np.concatenate([xq, xk, xv], -1)], 0)  # [4, C]
    z = O.silu(np.sum(win.T * w, axis=1))
    kh = z[dk:2 * dk] / np.sqrt(np.sum(z[dk:2 * dk] ** 2))
    for h in range(Hv):
        np.testing.assert_allclose(S[0, h] @ kh, z[2 * dk + h * dv: 2 * dk + (h + 1) * dv],
                                   rtol=1e-12, atol=1e-12)
        assert np.max(np.abs(S0[0, h] @ kh - S[0, h] @ kh)) > 0.1  # the old content was replaced
    np.testing.assert_array_equal(out, 0.0)  # gate 0: silu(0) = 0
