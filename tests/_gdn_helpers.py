"""Shared helpers of the parity tests: stage inputs from the oracle, head
slicing for sampled full-size checks, and the tolerance check.

The tolerance (max-abs error relative to the largest reference magnitude)
is 1e-4 for FP32 workloads and 2e-2 for BF16/FP16 ones, per output tensor.
"""
from __future__ import annotations

import numpy as np
import torch

from linear_attention_rnn_qkv_amd import synth
from oracle import gdn as O

TAU = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
f64 = synth.to_f64


def cu_of(x):
    return None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu().numpy().astype(np.int64)


def to_dev(x: dict, device="cuda") -> dict:
    out = {}
    for k, v in x.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    if x.get("proj") is not None:  # keep the views into one device buffer
        proj = x["proj"].to(device)
        base = x["proj"]
        for k in ("x_q", "x_k", "x_v", "gate", "b", "a"):
            v = x[k]
            off = v.storage_offset() - base.storage_offset()
            out[k] = proj.as_strided(v.shape, v.stride(), proj.storage_offset() + off)
        out["proj"] = proj
    return out


def assert_close(got, ref, tau, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= tau * scale, f"{what}: max|err| {err:.3e} > {tau:g} * max|ref| {scale:.3e}"
    return err / scale if scale else 0.0


def oracle_prologue(x, s: synth.Spec):
    """Oracle qkv (rounded to act), g, beta (rounded to f32) in float64."""
    xc = np.concatenate([f64(x["x_q"]), f64(x["x_k"]), f64(x["x_v"])], -1)
    qkv = O.round_to(O.causal_conv_silu(xc, f64(x["conv_w"]), f64(x["conv_b"]), cu_of(x)), s.act)
    beta, g = O.beta_and_g(f64(x["b"]), f64(x["a"]), f64(x["A_log"]), f64(x["dt_bias"]))
    return qkv, O.round_to(g, "f32"), O.round_to(beta, "f32")


def split_qkv(qkv, s: synth.Spec):
    B, T, _ = qkv.shape
    nq = s.Hqk * s.dk
    return (qkv[..., :nq].reshape(B, T, s.Hqk, s.dk), qkv[..., nq:2 * nq].reshape(B, T, s.Hqk, s.dk),
            qkv[..., 2 * nq:].reshape(B, T, s.Hv, s.dv))


def oracle_layer(x, s: synth.Spec, scale, use_l2=True, rms_eps=1e-5, return_stages=False):
    return O.layer(f64(x["x_q"]), f64(x["x_k"]), f64(x["x_v"]), f64(x["conv_w"]), f64(x["conv_b"]),
                   f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]), f64(x["gate"]),
                   f64(x["norm_w"]), Hqk=s.Hqk, dk=s.dk, Hv=s.Hv, dv=s.dv, act=s.act, scale=scale,
                   cu_seqlens=cu_of(x), use_qk_l2norm=use_l2, rms_eps=rms_eps,
                   return_stages=return_stages)


def slice_heads(x, s: synth.Spec, qk_heads):
    """Inputs restricted to query/key heads ``qk_heads`` and the value heads
    that read them (heads are independent, so the oracle of the slice equals
    the slice of the oracle). Returns (dict of float64 arrays, spec, v_heads)."""
    G = s.Hv // s.Hqk
    v_heads = [h for j in qk_heads for h in range(j * G, (j + 1) * G)]
    nq = s.Hqk * s.dk
    qc = np.concatenate([np.arange(j * s.dk, (j + 1) * s.dk) for j in qk_heads])
    vc = np.concatenate([np.arange(h * s.dv, (h + 1) * s.dv) for h in v_heads])
    w = x["conv_w"].cpu()
    out = {
        "x_q": f64(x["x_q"].cpu()[..., qc]), "x_k": f64(x["x_k"].cpu()[..., qc]),
        "x_v": f64(x["x_v"].cpu()[..., vc]),
        "conv_w": f64(torch.cat([w[qc], w[nq + qc], w[2 * nq + vc]])), "conv_b": None,
        "a": f64(x["a"].cpu()[..., v_heads]), "b": f64(x["b"].cpu()[..., v_heads]),
        "A_log": f64(x["A_log"].cpu()[v_heads]), "dt_bias": f64(x["dt_bias"].cpu()[v_heads]),
        "gate": f64(x["gate"].cpu()[:, :, v_heads]), "norm_w": f64(x["norm_w"].cpu()),
        "cu_seqlens": x["cu_seqlens"],
    }
    return out, s.replace(Hqk=len(qk_heads), Hv=len(v_heads)), v_heads


def oracle_layer_arrays(xa, s: synth.Spec, scale, threads=None):
    return O.layer(xa["x_q"], xa["x_k"], xa["x_v"], xa["conv_w"], None, xa["a"], xa["b"], xa["A_log"],
                   xa["dt_bias"], xa["gate"], xa["norm_w"], Hqk=s.Hqk, dk=s.dk, Hv=s.Hv, dv=s.dv,
                   act=s.act, scale=scale, cu_seqlens=cu_of(xa), threads=threads)
