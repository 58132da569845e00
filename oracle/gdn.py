"""FP64 CPU oracle for the Gated DeltaNet (GDN) layer core, forward only.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports it, and the two share
no code: the only thing both sides consume is the seeded input generator,
which holds none of the method's arithmetic.

Everything here is the plain definition, in float64, of what each step
computes, written from these pages:

* P1 - Megatron-LM pull request "perf(gated_delta_net): fold q/k L2-norm into
  the gated_delta_rule kernel" (sections What, Why, Validation).
* P2 - Megatron Core developer guide, "GDN Elementwise Fusion" (option table,
  "Post-GDR requirements", "Execution and numerical behavior").
* P3 - flash-linear-attention pull request "fused q/k/v short conv" for
  GatedDeltaNet (Summary, Why, Test plan, Risk / scope).

The recurrence formula itself is not printed on the pages; the reading taken
is the gated delta rule of Gated DeltaNet (Yang, Kautz and Hatamizadeh, ICLR
2025), see ``gdn_oracle.c``. Every place where the pages are silent carries a
``Reading:`` note.

Inputs are numpy float64 arrays holding the exact values of the stored
(possibly bf16/fp16) tensors. Stage outputs are rounded to their storage dtype
with ``round_to`` exactly where the layer materialises them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C recurrence with gcc (no fast-math: IEEE FP64)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        f = lib.oracle_gated_delta_rule
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        f.argtypes = [dp, dp, dp, dp, dp, ctypes.POINTER(i64), i64, i64, i64, i64,
                      i64, ctypes.c_double, dp, dp, dp, i64, ctypes.c_int]
        f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# --------------------------------------------------------------------------
# Rounding to a storage dtype (round to nearest, ties to even).
# --------------------------------------------------------------------------
_FMT = {  # significant bits p, exponent of the smallest normal, largest finite
    "f32": (24, -126, float(np.finfo(np.float32).max)),
    "bf16": (8, -126, (2.0 - 2.0 ** -7) * 2.0 ** 127),
    "f16": (11, -14, 65504.0),
}


def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest ``dtype`` value, ties to even.

    Plain definition: the spacing of representable numbers around |x| is
    2**(e - p) for |x| in [2**(e-1), 2**e) in the normal range and the
    subnormal spacing below it; ``np.round`` rounds half to even, and scaling
    by a power of two is exact in float64. Values beyond the largest finite
    number become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    p, emin, vmax = _FMT[dtype]
    out = np.zeros_like(x)
    nz = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[nz])  # x = m * 2**e with 0.5 <= |m| < 1
    ulp_exp = np.maximum(e, emin + 1) - p
    scale = np.ldexp(1.0, -ulp_exp)
    r = np.round(x[nz] * scale) / scale
    r[np.abs(r) > vmax] = np.inf * np.sign(r[np.abs(r) > vmax])
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    out[x == 0] = x[x == 0]
    return out


# --------------------------------------------------------------------------
# Prologue: concatenated depthwise causal conv + SiLU, beta and g.
# --------------------------------------------------------------------------
def silu(x):
    """x * sigmoid(x) in float64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def causal_conv_silu(x, w, bias=None, cu_seqlens=None):
    """Depthwise causal conv1d over the channel axis, then SiLU.

    P3 (Summary, Why): the q/k/v projections are concatenated along the
    channel axis and run through one depthwise ``causal_conv1d`` with the
    concatenated weights (and bias, if any); being depthwise, this is the same
    as three separate convolutions.

    x: [B, T, C]; w: [C, K]; bias: [C] or None. Reading: tap j of K
    multiplies token t - (K - 1) + j, so the last tap sees the current token;
    history before each sequence start is zero; bias is added before SiLU.
    With ``cu_seqlens`` (B must be 1) every sequence [cu[n], cu[n+1]) starts
    with zero history. Returns float64 [B, T, C] (not rounded).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, C = x.shape
    K = w.shape[1]
    if cu_seqlens is None:
        bounds = [(b, 0, T) for b in range(B)]
    else:
        assert B == 1
        cu = [int(c) for c in cu_seqlens]
        bounds = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    y = np.zeros_like(x)
    for b, t0, t1 in bounds:
        xs = x[b, t0:t1]  # one sequence
        L = t1 - t0
        acc = np.zeros((L, C))
        if bias is not None:
            acc += np.asarray(bias, dtype=np.float64)[None, :]
        for j in range(K):
            lag = K - 1 - j  # tap j reads token t - lag
            if lag >= L:
                continue
            acc[lag:] += w[None, :, j] * xs[: L - lag]
        y[b, t0:t1] = acc
    return silu(y)


def softplus(x):
    """log(1 + e^x). Reading: exact form, with x returned as is above 20."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return np.where(x > 20.0, x, np.log1p(np.exp(np.minimum(x, 20.0))))


def beta_and_g(b, a, A_log, dt_bias):
    """beta = sigmoid(b); g = -exp(A_log[h]) * softplus(a + dt_bias[h]).

    P2 (option table) lists "beta and decay preparation" among the pre-recurrence
    fused operations without formulas. Reading: the Gated DeltaNet
    parameterisation (write strength beta in (0, 1), log-decay g < 0). b, a:
    [..., Hv]; A_log, dt_bias: [Hv]. Returns float64 (beta, g).
    """
    b = np.asarray(b, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        beta = 1.0 / (1.0 + np.exp(-b))
    g = -np.exp(np.asarray(A_log, dtype=np.float64)) * softplus(
        a + np.asarray(dt_bias, dtype=np.float64))
    return beta, g


# --------------------------------------------------------------------------
# q/k L2 normalisation.
# --------------------------------------------------------------------------
def l2norm(x, eps: float = 1e-6):
    """x / sqrt(sum(x^2) + eps) over the last dim.

    P1 (Why): per head over the last dimension, eps 1e-6 on both the caller
    side and the in-kernel route. Reading: eps is added to the sum of squares
    inside the square root.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


# --------------------------------------------------------------------------
# The recurrence.
# --------------------------------------------------------------------------
def gated_delta_rule(q, k, v, g, beta, scale=1.0, use_qk_l2norm=True,
                     l2_eps=1e-6, cu_seqlens=None, initial_state=None,
                     output_final_state=False, threads=None, rows_per_unit=16):
    """Sequential token-by-token gated delta rule (FP64, C, threads).

    q, k: [B, T, Hqk, dk]; v: [B, T, Hv, dv]; g, beta: [B, T, Hv].
    Dense when ``cu_seqlens`` is None (each batch row is one sequence);
    packed when given (B == 1, state restarts at every boundary).
    ``use_qk_l2norm`` normalises q and k first (P1: the kernel flag
    use_qk_l2norm_in_kernel; off is a no-op). Value head h reads q/k head
    h // (Hv // Hqk) (P1 Why: per-head normalisation makes head replication
    result-neutral; reading: heads repeated in consecutive groups).
    initial_state / final state: [N, Hv, dv, dk]. Returns o [B, T, Hv, dv]
    float64 (not rounded) and the final state (or None).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if use_qk_l2norm:
        q = l2norm(q, l2_eps)
        k = l2norm(k, l2_eps)
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        assert B == 1
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    qf = np.ascontiguousarray(q.reshape(B * T, Hqk, dk))
    kf = np.ascontiguousarray(k.reshape(B * T, Hqk, dk))
    vf = np.ascontiguousarray(v.reshape(B * T, Hv, dv))
    gf = np.ascontiguousarray(np.asarray(g, dtype=np.float64).reshape(B * T, Hv))
    bf = np.ascontiguousarray(np.asarray(beta, dtype=np.float64).reshape(B * T, Hv))
    o = np.zeros((B * T, Hv, dv))
    init = None
    if initial_state is not None:
        init = np.ascontiguousarray(np.asarray(initial_state, dtype=np.float64))
        assert init.shape == (N, Hv, dv, dk)
    fin = np.zeros((N, Hv, dv, dk)) if output_final_state else None
    if B * T > 0:
        lib = _load()
        dp = ctypes.POINTER(ctypes.c_double)

        def P(a):
            return None if a is None else a.ctypes.data_as(dp)

        rc = lib.oracle_gated_delta_rule(
            P(qf), P(kf), P(vf), P(gf), P(bf),
            cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, Hqk, Hv, dk, dv,
            float(scale), P(init), P(o), P(fin), int(rows_per_unit),
            int(threads or default_threads()))
        if rc != 0:
            raise RuntimeError(f"oracle_gated_delta_rule failed ({rc})")
    elif fin is not None and init is not None:
        fin[...] = init
    return o.reshape(B, T, Hv, dv), fin


# --------------------------------------------------------------------------
# Post-recurrence: output RMSNorm, then the SiLU gate.
# --------------------------------------------------------------------------
def gated_rmsnorm(o, gate, weight, eps: float = 1e-5, act: str = "bf16"):
    """RMSNorm over head_dim, materialised in the activation dtype, then gate.

    P2 (option table; Execution and numerical behavior): output RMSNorm and
    SiLU gating; the activation-dtype RMSNorm result is materialised before
    the SiLU-gate multiply, which is done in FP32. Readings: weight multiplies
    directly (not 1 + w); eps is a parameter (1e-5 by default); the output is
    in the activation dtype. The oracle evaluates the gate product in float64
    and rounds once, which agrees with an FP32 product rounded to a 16-bit
    dtype except at rounding ties.
    o, gate: [..., dv]; weight: [dv]. Returns float64 values of ``act``.
    """
    o = np.asarray(o, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    y = round_to(o * r * np.asarray(weight, dtype=np.float64), act)
    return round_to(y * silu(gate), act)


# --------------------------------------------------------------------------
# The layer core: prologue -> recurrence -> gated norm.
# --------------------------------------------------------------------------
def layer(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, *,
          Hqk, dk, Hv, dv, act, scale, cu_seqlens=None, use_qk_l2norm=True,
          l2_eps=1e-6, rms_eps=1e-5, threads=None, return_stages=False):
    """The whole forward layer core with the layer's materialisation points.

    x_q [B,T,Hqk*dk], x_k [B,T,Hqk*dk], x_v [B,T,Hv*dv]; conv_w [C,4];
    a, b [B,T,Hv]; A_log, dt_bias [Hv]; gate [B,T,Hv,dv]; norm_w [dv].
    Reading of the storage points: conv output in the activation dtype, g and
    beta in FP32, recurrence output in the activation dtype, RMSNorm result
    and final output in the activation dtype.
    """
    x = np.concatenate([np.asarray(x_q, np.float64), np.asarray(x_k, np.float64),
                        np.asarray(x_v, np.float64)], axis=-1)
    B, T, C = x.shape
    qkv = round_to(causal_conv_silu(x, conv_w, conv_b, cu_seqlens), act)
    nq = Hqk * dk
    q = qkv[..., :nq].reshape(B, T, Hqk, dk)
    k = qkv[..., nq:2 * nq].reshape(B, T, Hqk, dk)
    v = qkv[..., 2 * nq:].reshape(B, T, Hv, dv)
    beta, g = beta_and_g(b, a, A_log, dt_bias)
    beta = round_to(beta, "f32")
    g = round_to(g, "f32")
    o, _ = gated_delta_rule(q, k, v, g, beta, scale=scale,
                            use_qk_l2norm=use_qk_l2norm, l2_eps=l2_eps,
                            cu_seqlens=cu_seqlens, threads=threads)
    o = round_to(o, act)
    out = gated_rmsnorm(o, gate, norm_w, rms_eps, act)
    if return_stages:
        return out, dict(qkv=qkv, g=g, beta=beta, o=o)
    return out


# --------------------------------------------------------------------------
# Recurrent decode: one new token per sequence with a conv cache and a state.
# --------------------------------------------------------------------------
def decode_step(x_q, x_k, x_v, conv_w, conv_b, conv_state, a, b, A_log, dt_bias,
                state, gate, norm_w, *, Hqk, dk, Hv, dv, act, scale,
                use_qk_l2norm=True, l2_eps=1e-6, rms_eps=1e-5):
    """One token of the layer core for each of N independent sequences.

    The recurrent form of the same layer (Gated DeltaNet's gated delta rule,
    one token; the conv of P3 Summary evaluated at the newest token; the gated
    norm of P2 Execution and numerical behavior). Reading of the cache: the
    conv keeps the last K-1 = 3 inputs of every channel, oldest first, in the
    activation dtype; a fresh sequence has a zero cache and a zero state, so T
    steps from zero reproduce ``layer`` over those T tokens.

    x_q, x_k [N, Hqk*dk]; x_v [N, Hv*dv]; conv_w [C, 4]; conv_state [N, 3, C];
    a, b [N, Hv]; state [N, Hv, dv, dk] (FP32 values); gate [N, Hv, dv].
    Returns (out [N, Hv, dv] float64 values of ``act``, the new conv cache
    [N, 3, C], the new state [N, Hv, dv, dk] float64, not rounded).
    """
    x = np.concatenate([np.asarray(x_q, np.float64), np.asarray(x_k, np.float64),
                        np.asarray(x_v, np.float64)], axis=-1)  # [N, C]
    cache = np.asarray(conv_state, np.float64)
    N, C = x.shape
    w = np.asarray(conv_w, np.float64)
    # the window of the newest token: three cached inputs then the new one;
    # tap j multiplies window entry j
    window = np.concatenate([cache, x[:, None, :]], axis=1)  # [N, 4, C]
    y = np.einsum("njc,cj->nc", window, w)
    if conv_b is not None:
        y = y + np.asarray(conv_b, np.float64)[None, :]
    z = round_to(silu(y), act)
    new_cache = window[:, 1:, :].copy()
    nq = Hqk * dk
    q = z[:, :nq].reshape(N, Hqk, dk)
    k = z[:, nq:2 * nq].reshape(N, Hqk, dk)
    v = z[:, 2 * nq:].reshape(N, Hv, dv)
    beta, g = beta_and_g(b, a, A_log, dt_bias)
    beta = round_to(beta, "f32")
    g = round_to(g, "f32")
    if use_qk_l2norm:
        q, k = l2norm(q, l2_eps), l2norm(k, l2_eps)
    G = Hv // Hqk
    S = np.array(state, dtype=np.float64, copy=True)
    o = np.zeros((N, Hv, dv))
    for n in range(N):
        for h in range(Hv):
            kk, qq = k[n, h // G], q[n, h // G]
            # S_t = e^g S_{t-1} (I - beta k k^T) + beta v k^T;  o = scale S_t q
            Sd = np.exp(g[n, h]) * S[n, h]
            S[n, h] = Sd - beta[n, h] * np.outer(Sd @ kk, kk) + beta[n, h] * np.outer(v[n, h], kk)
            o[n, h] = scale * (S[n, h] @ qq)
    o = round_to(o, act)
    out = gated_rmsnorm(o, gate, norm_w, rms_eps, act)
    return out, new_cache, S
