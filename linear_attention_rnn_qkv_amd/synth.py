"""Seeded synthetic inputs for the GDN layer core.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle may consume what it
produces.

Workloads (shapes of the pages' layer: flash-linear-attention's GatedDeltaNet
with num_heads=6 and expand_v=2 in the fused-conv pull request's benchmark, and
the long-context grouped-query shapes of the Megatron pull requests):

  id  name                 act   gate          B   tokens        Hqk x dk  Hv x dv
  0   tiny-fp32            f32   f32           1   128           6 x 64    6 x 128
  1   bf16-B2-T2048-hd256  bf16  bf16 (view)   2   2 x 2048      6 x 256   6 x 512
  2   gqa-bf16-T8192       bf16  f32           1   8192          16 x 128  32 x 128
  3   long-bf16-T131072    bf16  bf16          1   131072        16 x 128  32 x 128
  4   varlen-fp16-64seq    f16   f16           1   64 packed     16 x 128  32 x 128

Value distributions (all workloads): pre-conv q/k/v, gate, a and b ~ N(0, 1);
conv weight ~ U(-0.5, 0.5), shape [C, 4], no bias; A_log = log U(1, 16);
dt_bias ~ N(0, 0.1); RMSNorm weight ~ 1 + N(0, 0.02). Draws are made in
float32 with ``numpy.random.default_rng(42 + id)`` in a fixed order and cast
to each tensor's dtype with round-to-nearest-even (torch's conversion).
Workload 1 draws one projection buffer [2, 2048, 9228] laid out
[q 1536 | k 1536 | v 3072 | gate 3072 | b 6 | a 6] and hands out strided views
into it (row pitch 18456 bytes, 8 mod 16). Workload 4 draws its 64 sequence
lengths from ``default_rng(42).integers(1, 4097, size=64)``.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Spec:
    name: str
    act: str
    gate_dtype: str
    w_dtype: str
    B: int
    T: int                      # tokens per row (packed total when varlen)
    Hqk: int
    dk: int
    Hv: int
    dv: int
    seed: int
    lengths: Optional[Tuple[int, ...]] = None   # packed sequences (B == 1)
    gate_in_proj: bool = False                  # gate etc. are views of one buffer
    K: int = 4                                  # conv taps

    @property
    def C(self) -> int:
        return 2 * self.Hqk * self.dk + self.Hv * self.dv

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def n_seqs(self) -> int:
        return len(self.lengths) if self.lengths is not None else self.B

    def replace(self, **kw) -> "Spec":
        if "lengths" in kw and kw["lengths"] is not None:
            kw["lengths"] = tuple(int(x) for x in kw["lengths"])
            kw.setdefault("T", int(sum(kw["lengths"])))
        return dataclasses.replace(self, **kw)


def _varlen_lengths() -> Tuple[int, ...]:
    return tuple(int(x) for x in np.random.default_rng(42).integers(1, 4097, size=64))


def spec(cfg: int) -> Spec:
    if cfg == 0:
        return Spec("tiny-fp32", "f32", "f32", "f32", 1, 128, 6, 64, 6, 128, 42)
    if cfg == 1:
        return Spec("bf16-B2-T2048-hd256", "bf16", "bf16", "bf16", 2, 2048, 6, 256,
                    6, 512, 43, gate_in_proj=True)
    if cfg == 2:
        return Spec("gqa-bf16-T8192", "bf16", "f32", "f32", 1, 8192, 16, 128, 32,
                    128, 44)
    if cfg == 3:
        return Spec("long-bf16-T131072", "bf16", "bf16", "bf16", 1, 131072, 16,
                    128, 32, 128, 45)
    if cfg == 4:
        L = _varlen_lengths()
        return Spec("varlen-fp16-64seq", "f16", "f16", "f16", 1, int(sum(L)), 16,
                    128, 32, 128, 46, lengths=L)
    raise ValueError(f"unknown workload {cfg}")


def _cast(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(TORCH_DTYPE[dtype])


def make_inputs(s: Spec, device="cpu", dt_bias_override=None) -> dict:
    """Draw every input of the layer core for workload ``s``.

    Returns a dict of torch tensors on ``device``: x_q, x_k [B,T,Hqk*dk],
    x_v [B,T,Hv*dv], a, b [B,T,Hv], gate [B,T,Hv,dv] (views into ``proj``
    when ``s.gate_in_proj``), conv_w [C,4] (act dtype), conv_b (None),
    A_log, dt_bias [Hv] (f32), norm_w [dv], cu_seqlens (int32 [N+1] or None).
    ``dt_bias_override`` replaces the dt_bias draw (stress sets).
    """
    rng = np.random.default_rng(s.seed)
    B, T = s.B, s.T
    nq, nv = s.Hqk * s.dk, s.Hv * s.dv
    out = {}
    if s.gate_in_proj:
        width = 2 * nq + 2 * nv + 2 * s.Hv
        proj = _cast(rng.standard_normal((B, T, width), dtype=np.float32), s.act, device)
        o = 0
        out["x_q"] = proj[..., o:o + nq]; o += nq
        out["x_k"] = proj[..., o:o + nq]; o += nq
        out["x_v"] = proj[..., o:o + nv]; o += nv
        out["gate"] = proj[..., o:o + nv].unflatten(-1, (s.Hv, s.dv)); o += nv
        out["b"] = proj[..., o:o + s.Hv]; o += s.Hv
        out["a"] = proj[..., o:o + s.Hv]; o += s.Hv
        out["proj"] = proj
    else:
        out["x_q"] = _cast(rng.standard_normal((B, T, nq), dtype=np.float32), s.act, device)
        out["x_k"] = _cast(rng.standard_normal((B, T, nq), dtype=np.float32), s.act, device)
        out["x_v"] = _cast(rng.standard_normal((B, T, nv), dtype=np.float32), s.act, device)
        out["gate"] = _cast(rng.standard_normal((B, T, s.Hv, s.dv), dtype=np.float32),
                            s.gate_dtype, device)
        out["b"] = _cast(rng.standard_normal((B, T, s.Hv), dtype=np.float32), s.act, device)
        out["a"] = _cast(rng.standard_normal((B, T, s.Hv), dtype=np.float32), s.act, device)
        out["proj"] = None
    out["conv_w"] = _cast(rng.uniform(-0.5, 0.5, (s.C, s.K)).astype(np.float32), s.act, device)
    out["conv_b"] = None
    out["A_log"] = _cast(np.log(rng.uniform(1.0, 16.0, s.Hv)).astype(np.float32), "f32", device)
    dtb = rng.normal(0.0, 0.1, s.Hv).astype(np.float32)
    if dt_bias_override is not None:
        dtb = np.asarray(dt_bias_override, dtype=np.float32)
    out["dt_bias"] = _cast(dtb, "f32", device)
    out["norm_w"] = _cast((1.0 + rng.normal(0.0, 0.02, s.dv)).astype(np.float32),
                          s.w_dtype, device)
    if s.lengths is not None:
        cu = np.zeros(len(s.lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(s.lengths)
        out["cu_seqlens"] = torch.from_numpy(cu).to(device)
    else:
        out["cu_seqlens"] = None
    return out


def stress_dt_bias(Hv: int) -> np.ndarray:
    """Stress set S1: dt_bias spread from -12 to 0 across heads, so per-head
    state half-lives range from about one token to about 1e5 tokens."""
    if Hv == 1:
        return np.array([-12.0], dtype=np.float32)
    return (-12.0 + 12.0 * np.arange(Hv) / (Hv - 1)).astype(np.float32)


def to_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact float64 copy of a (possibly 16-bit) tensor, on the host."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
