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
float32 from ``numpy.random.SeedSequence(42 + id)``: tensor number i (in a
fixed order) uses child i of that sequence, and large tensors are drawn in
blocks of rows, block j from child j of the tensor's sequence, so that blocks
can be drawn on several threads with a result that does not depend on the
thread count. Values are cast to each tensor's dtype with round-to-nearest-
even (torch's conversion).
Workload 1 draws one projection buffer [2, 2048, 9228] laid out
[q 1536 | k 1536 | v 3072 | gate 3072 | b 6 | a 6] and hands out strided views
into it (row pitch 18456 bytes, 8 mod 16). Workload 4 draws its 64 sequence
lengths from ``default_rng(42).integers(1, 4097, size=64)``.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
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
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DTYPE[dtype]).to(device=device)


_BLOCK = 1 << 20  # values per independently seeded block


class _Draws:
    """Tensor-by-tensor draws from one SeedSequence (see module docstring)."""

    def __init__(self, seed: int):
        self.seq = np.random.SeedSequence(seed)
        self.n = 0

    def _next(self) -> np.random.SeedSequence:
        child = self.seq.spawn(1)[0]
        self.n += 1
        return child

    def normal(self, shape) -> np.ndarray:
        seq = self._next()
        shape = tuple(int(x) for x in shape)
        total = int(np.prod(shape)) if shape else 1
        out = np.empty(total, dtype=np.float32)
        nblk = max(1, (total + _BLOCK - 1) // _BLOCK)
        kids = seq.spawn(nblk)

        def fill(j):
            lo, hi = j * _BLOCK, min(total, (j + 1) * _BLOCK)
            np.random.default_rng(kids[j]).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

        workers = min(nblk, max(1, min(16, os.cpu_count() or 1)))
        if workers == 1:
            for j in range(nblk):
                fill(j)
        else:
            with cf.ThreadPoolExecutor(workers) as ex:
                list(ex.map(fill, range(nblk)))
        return out.reshape(shape)

    def rng(self) -> np.random.Generator:
        return np.random.default_rng(self._next())


def make_inputs(s: Spec, device="cpu", dt_bias_override=None) -> dict:
    """Draw every input of the layer core for workload ``s``.

    Returns a dict of torch tensors on ``device``: x_q, x_k [B,T,Hqk*dk],
    x_v [B,T,Hv*dv], a, b [B,T,Hv], gate [B,T,Hv,dv] (views into ``proj``
    when ``s.gate_in_proj``), conv_w [C,4] (act dtype), conv_b (None),
    A_log, dt_bias [Hv] (f32), norm_w [dv], cu_seqlens (int32 [N+1] or None).
    ``dt_bias_override`` replaces the dt_bias draw (stress sets).
    """
    dr = _Draws(s.seed)
    B, T = s.B, s.T
    nq, nv = s.Hqk * s.dk, s.Hv * s.dv
    out = {}
    if s.gate_in_proj:
        width = 2 * nq + 2 * nv + 2 * s.Hv
        proj = _cast(dr.normal((B, T, width)), s.act, device)
        o = 0
        out["x_q"] = proj[..., o:o + nq]; o += nq
        out["x_k"] = proj[..., o:o + nq]; o += nq
        out["x_v"] = proj[..., o:o + nv]; o += nv
        out["gate"] = proj[..., o:o + nv].unflatten(-1, (s.Hv, s.dv)); o += nv
        out["b"] = proj[..., o:o + s.Hv]; o += s.Hv
        out["a"] = proj[..., o:o + s.Hv]; o += s.Hv
        out["proj"] = proj
    else:
        out["x_q"] = _cast(dr.normal((B, T, nq)), s.act, device)
        out["x_k"] = _cast(dr.normal((B, T, nq)), s.act, device)
        out["x_v"] = _cast(dr.normal((B, T, nv)), s.act, device)
        out["gate"] = _cast(dr.normal((B, T, s.Hv, s.dv)),
                            s.gate_dtype, device)
        out["b"] = _cast(dr.normal((B, T, s.Hv)), s.act, device)
        out["a"] = _cast(dr.normal((B, T, s.Hv)), s.act, device)
        out["proj"] = None
    rng = dr.rng()
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


def randn(shape, dtype: str, seed: int, device="cpu") -> torch.Tensor:
    """Seeded N(0, 1) draws of ``shape`` cast to ``dtype`` (stand-alone stage
    inputs, e.g. a recurrence output fed to the gated norm on its own)."""
    return _cast(_Draws(seed).normal(shape), dtype, device)


def uniform(shape, lo: float, hi: float, seed: int) -> np.ndarray:
    """Seeded U(lo, hi) float64 draws (stress sets of the recurrence)."""
    return np.random.default_rng(seed).uniform(lo, hi, shape)
