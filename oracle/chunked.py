"""FP64 chunked evaluation of the gated delta rule (any chunk size).

TEST INFRASTRUCTURE, used only by the tests: it exists to show, in float64 and
against the sequential oracle, that the chunk algebra which a chunked kernel
evaluates reaches the same result as the token-by-token recurrence. The HIP
kernels do not use it and it does not use them.

The pages name the chunked mode (FLA ``chunk_gated_delta_rule``, flash-linear-
attention pull request on the fused q/k/v short conv, Benchmark section) but do
not give the algorithm. Reading: the WY / UT-transform form of the delta rule
(Yang et al., "Parallelizing Linear Transformers with the Delta Rule over
Sequence Length", NeurIPS 2024) with the gating of Gated DeltaNet (ICLR 2025).
Derivation, for one chunk of rows r = 0..C-1 entering with state S0 (dv x dk):

  gamma_r = g_0 + ... + g_r                          (within-chunk cumsum)
  A[r, i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i)      for i < r, else 0
  T       = (I + A)^-1                               (unit lower triangular)
  W       = T diag(beta exp(gamma)) K                (C x dk)
  U       = T diag(beta) V                           (C x dv)
  Vn      = U - W S0^T                               (C x dv, the new values)
  P[r, i] = exp(gamma_r - gamma_i) (q_r . k_i)             for i <= r
  O       = scale (diag(exp(gamma)) Q S0^T + P Vn)
  S_C     = exp(gamma_C) S0 + Vn^T diag(exp(gamma_C - gamma)) K

Only exponents gamma_r - gamma_i with i <= r, gamma_r and gamma_C - gamma_i
appear, all of which are <= 0 when every g <= 0.
"""
from __future__ import annotations

import numpy as np

from .gdn import l2norm


def chunk_step(Q, K, V, g, beta, S0, scale):
    """One chunk: returns (O [C, dv], S_end [dv, dk]). All float64."""
    C = Q.shape[0]
    gam = np.cumsum(g)
    diff = gam[:, None] - gam[None, :]  # gamma_r - gamma_i
    lower = np.tril(np.ones((C, C), dtype=bool), -1)
    A = np.where(lower, beta[:, None] * np.exp(np.where(lower, diff, 0.0)) * (K @ K.T), 0.0)
    T = np.linalg.solve(np.eye(C) + A, np.eye(C))
    W = T @ ((beta * np.exp(gam))[:, None] * K)
    U = T @ (beta[:, None] * V)
    Vn = U - W @ S0.T
    incl = np.tril(np.ones((C, C), dtype=bool))
    P = np.where(incl, np.exp(np.where(incl, diff, 0.0)) * (Q @ K.T), 0.0)
    O = scale * (np.exp(gam)[:, None] * (Q @ S0.T) + P @ Vn)
    S = np.exp(gam[-1]) * S0 + Vn.T @ (np.exp(gam[-1] - gam)[:, None] * K)
    return O, S


def chunked_gated_delta_rule(q, k, v, g, beta, scale=1.0, use_qk_l2norm=True,
                             l2_eps=1e-6, chunk=64, cu_seqlens=None,
                             initial_state=None):
    """Same signature and result as ``gdn.gated_delta_rule`` (FP64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    if use_qk_l2norm:
        q, k = l2norm(q, l2_eps), l2norm(k, l2_eps)
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = Hv // Hqk
    if cu_seqlens is None:
        segs = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(c) for c in cu_seqlens]
        segs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    o = np.zeros((B, T, Hv, dv))
    fin = np.zeros((len(segs), Hv, dv, dk))
    for n, (b, t0, t1) in enumerate(segs):
        for h in range(Hv):
            S = (np.zeros((dv, dk)) if initial_state is None
                 else np.array(initial_state[n, h], dtype=np.float64))
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                O, S = chunk_step(q[b, c0:c1, h // G], k[b, c0:c1, h // G],
                                  v[b, c0:c1, h], g[b, c0:c1, h],
                                  beta[b, c0:c1, h], S, scale)
                o[b, c0:c1, h] = O
            fin[n, h] = S
    return o, fin
