"""Thin ctypes binding of ``libgdn.so`` (the C ABI in ``include/gdn.h``).

Argument marshalling only: torch tensors are turned into ``gdn_tensor``
descriptors (device pointer, dtype, shape, element strides), outputs the
caller does not pass are allocated with torch, and the call is enqueued on
torch's current HIP stream. Every step of the computation runs in the HIP
kernels of the library; there is no other path. If the library is missing the
import of any function here raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_ERR_INVALID_VALUE, GDN_ERR_NOT_SUPPORTED, GDN_ERR_LAUNCH = 0, 1, 2, 3
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20  # static chunk scratch of gdn_chunk_rule_fwd_noalloc (gdn.h)
DTYPE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2, torch.int32: 3}
_NAMES = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


class GdnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 5), ("stride", ctypes.c_int64 * 5)]


class GdnDims(ctypes.Structure):
    _fields_ = [("Hqk", ctypes.c_int64), ("dk", ctypes.c_int64), ("Hv", ctypes.c_int64),
                ("dv", ctypes.c_int64)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[gdn status {status}] {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_attention_rnn_qkv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(GdnTensor)
        vp, f32, i32 = ctypes.c_void_p, ctypes.c_float, ctypes.c_int32
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_version.restype = ctypes.c_char_p
        L.gdn_prologue_fwd.argtypes = [P] * 10 + [ctypes.POINTER(GdnDims), i32, f32, P, P, P, vp]
        L.gdn_chunk_rule_fwd.argtypes = [P, P, P, P, P, f32, i32, f32, P, P, P, P, vp, ctypes.c_size_t, vp]
        L.gdn_chunk_rule_fwd_noalloc.argtypes = [P, P, P, P, P, f32, i32, f32, P, P, P, P, vp]
        L.gdn_chunk_rule_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                     ctypes.POINTER(GdnDims), i32]
        L.gdn_chunk_rule_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_gated_norm_fwd.argtypes = [P, P, P, f32, P, vp]
        L.gdn_layer_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.POINTER(GdnDims), i32]
        L.gdn_layer_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_layer_fwd.argtypes = ([P] * 12 + [ctypes.POINTER(GdnDims), f32, i32, f32, f32, vp,
                                                ctypes.c_size_t, P, vp])
        L.gdn_decode_fwd.argtypes = ([P] * 11 + [ctypes.POINTER(GdnDims), f32, i32, f32, P, P, f32, P, vp])
        L.gdn_gated_norm_bwd_workspace_bytes.argtypes = [ctypes.c_int64] * 4
        L.gdn_gated_norm_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_gated_norm_bwd.argtypes = [P, P, P, f32, P, P, P, P, vp, ctypes.c_size_t, vp]
        L.gdn_prologue_bwd_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(GdnDims)]
        L.gdn_prologue_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_prologue_bwd.argtypes = [P] * 10 + [ctypes.POINTER(GdnDims)] + [P] * 12 + [vp, ctypes.c_size_t, vp]
        L.gdn_chunk_rule_bwd_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                         ctypes.POINTER(GdnDims)]
        L.gdn_chunk_rule_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_chunk_rule_bwd.argtypes = [P] * 5 + [f32, i32, f32] + [P] * 10 + [vp, ctypes.c_size_t, vp]
        L.gdn_layer_bwd_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                    ctypes.POINTER(GdnDims), i32]
        L.gdn_layer_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_layer_bwd.argtypes = ([P] * 12 + [ctypes.POINTER(GdnDims), f32, i32, f32, f32] + [P] * 12 +
                                    [vp, ctypes.c_size_t, vp])
        L.gdn_layer_bwd_saved.argtypes = L.gdn_layer_bwd.argtypes
        for name in ("gdn_prologue_fwd", "gdn_chunk_rule_fwd", "gdn_gated_norm_fwd", "gdn_layer_fwd",
                     "gdn_decode_fwd", "gdn_gated_norm_bwd", "gdn_prologue_bwd", "gdn_chunk_rule_bwd",
                     "gdn_layer_bwd", "gdn_layer_bwd_saved"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def desc(t: Optional[torch.Tensor]):
    """gdn_tensor descriptor of a tensor (None -> NULL)."""
    if t is None:
        return None
    if t.dtype not in DTYPE:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > 5:
        raise ValueError("at most 5 dims")
    d = GdnTensor()
    d.data = t.data_ptr() if t.numel() > 0 else 0
    d.dtype = DTYPE[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _p(d):
    return None if d is None else ctypes.byref(d)


def dims_of(Hqk: int, dk: int, Hv: int, dv: int) -> GdnDims:
    return GdnDims(Hqk, dk, Hv, dv)


def _stream(t: torch.Tensor):
    if t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(0)


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, lib().gdn_last_error().decode())


def gdn_last_error() -> str:
    return lib().gdn_last_error().decode()


def gdn_version() -> str:
    return lib().gdn_version().decode()


def gdn_prologue_fwd(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens,
                     dims: Sequence[int], caller_l2norm: bool = False, l2_eps: float = 1e-6,
                     out_qkv=None, out_g=None, out_beta=None):
    """Concatenated causal conv + SiLU and beta/g. Returns (qkv, g, beta)."""
    Hqk, dk, Hv, dv = dims
    B, T = x_q.shape[0], x_q.shape[1]
    C = 2 * Hqk * dk + Hv * dv
    dev = x_q.device
    if out_qkv is None:
        out_qkv = torch.empty((B, T, C), dtype=x_q.dtype, device=dev)
    if out_g is None:
        out_g = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
    if out_beta is None:
        out_beta = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
    D = [desc(t) for t in (x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens)]
    O = [desc(t) for t in (out_qkv, out_g, out_beta)]
    gd = dims_of(Hqk, dk, Hv, dv)
    _check(lib().gdn_prologue_fwd(*[_p(d) for d in D], ctypes.byref(gd), int(bool(caller_l2norm)),
                                  float(l2_eps), *[_p(d) for d in O], _stream(x_q)))
    return out_qkv, out_g, out_beta


def gdn_chunk_rule_workspace_bytes(B: int, T: int, dims: Sequence[int], dtype: torch.dtype,
                                   n_seqs: int = 0) -> int:
    gd = dims_of(*dims)
    return int(lib().gdn_chunk_rule_workspace_bytes(int(B), int(T), int(n_seqs), ctypes.byref(gd), DTYPE[dtype]))


def gdn_chunk_rule_fwd(q, k, v, g, beta, scale: float, use_qk_l2norm_in_kernel: bool = True,
                       l2_eps: float = 1e-6, cu_seqlens=None, initial_state=None, out_o=None,
                       output_final_state: bool = False, final_state=None, workspace="auto"):
    """Chunked gated delta rule. Returns (o, final_state or None).

    workspace: "auto" allocates the chunk workspace (two-kernel path where it
    applies), None passes none (single-kernel path), or a uint8 device tensor
    of at least gdn_chunk_rule_workspace_bytes(...) bytes."""
    B, T, Hv, dv = v.shape
    Hqk, dk = q.shape[2], q.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.shape[0] - 1
    if out_o is None:
        out_o = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, Hv, dv, dk), dtype=torch.float32, device=q.device)
    if isinstance(workspace, str):
        nb = gdn_chunk_rule_workspace_bytes(B, T, (Hqk, dk, Hv, dv), q.dtype,
                                            0 if cu_seqlens is None else N)
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb else None
    wptr = ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0)
    wlen = ctypes.c_size_t(workspace.numel() if workspace is not None else 0)
    D = [desc(t) for t in (q, k, v, g, beta)]
    E = [desc(t) for t in (cu_seqlens, initial_state, out_o, final_state)]
    _check(lib().gdn_chunk_rule_fwd(*[_p(d) for d in D], float(scale),
                                    int(bool(use_qk_l2norm_in_kernel)), float(l2_eps),
                                    *[_p(d) for d in E], wptr, wlen, _stream(q)))
    return out_o, final_state


def gdn_chunk_rule_fwd_noalloc(q, k, v, g, beta, scale: float, use_qk_l2norm_in_kernel: bool = True,
                               l2_eps: float = 1e-6, cu_seqlens=None, initial_state=None, out_o=None,
                               final_state=None):
    """gdn_chunk_rule_fwd with the chunk records in the library's static
    device scratch (the C call allocates nothing; outputs are the caller's).
    Returns (o, final_state or None)."""
    if out_o is None:
        out_o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    D = [desc(t) for t in (q, k, v, g, beta)]
    E = [desc(t) for t in (cu_seqlens, initial_state, out_o, final_state)]
    _check(lib().gdn_chunk_rule_fwd_noalloc(*[_p(d) for d in D], float(scale),
                                            int(bool(use_qk_l2norm_in_kernel)), float(l2_eps),
                                            *[_p(d) for d in E], _stream(q)))
    return out_o, final_state


def gdn_gated_norm_fwd(o, gate, weight, eps: float = 1e-5, out=None):
    """RMSNorm (act dtype) then FP32 SiLU gate. Returns out (contiguous)."""
    if out is None:
        out = torch.empty(o.shape, dtype=o.dtype, device=o.device)
    D = [desc(t) for t in (o, gate, weight)]
    _check(lib().gdn_gated_norm_fwd(*[_p(d) for d in D], float(eps), _p(desc(out)), _stream(o)))
    return out


def gdn_layer_workspace_bytes(B: int, T: int, dims: Sequence[int], dtype: torch.dtype,
                              n_seqs: int = 0) -> int:
    gd = dims_of(*dims)
    return int(lib().gdn_layer_workspace_bytes(int(B), int(T), int(n_seqs), ctypes.byref(gd), DTYPE[dtype]))


def gdn_layer_fwd(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, cu_seqlens,
                  dims: Sequence[int], scale: float, use_qk_l2norm_in_kernel: bool = True,
                  l2_eps: float = 1e-6, rms_eps: float = 1e-5, workspace=None, out=None):
    """The layer core (prologue -> chunk rule -> gated norm). Returns out."""
    Hqk, dk, Hv, dv = dims
    B, T = x_q.shape[0], x_q.shape[1]
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    nbytes = gdn_layer_workspace_bytes(B, T, dims, x_q.dtype, n_seqs)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x_q.device)
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=x_q.dtype, device=x_q.device)
    D = [desc(t) for t in (x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w,
                           cu_seqlens)]
    gd = dims_of(Hqk, dk, Hv, dv)
    _check(lib().gdn_layer_fwd(*[_p(d) for d in D], ctypes.byref(gd), float(scale),
                               int(bool(use_qk_l2norm_in_kernel)), float(l2_eps), float(rms_eps),
                               ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
                               _p(desc(out)), _stream(x_q)))
    return out


def gdn_decode_fwd(x_q, x_k, x_v, conv_w, conv_b, conv_state, a, b, A_log, dt_bias, state, gate,
                   norm_w, dims: Sequence[int], scale: float, use_qk_l2norm_in_kernel: bool = True,
                   l2_eps: float = 1e-6, rms_eps: float = 1e-5, out=None):
    """One decode step; conv_state [N,3,C] and state [N,Hv,dv,dk] are updated
    in place. Returns out [N, Hv, dv]."""
    Hqk, dk, Hv, dv = dims
    N = x_q.shape[0]
    if out is None:
        out = torch.empty((N, Hv, dv), dtype=x_q.dtype, device=x_q.device)
    D = [desc(t) for t in (x_q, x_k, x_v, conv_w, conv_b, conv_state, a, b, A_log, dt_bias, state)]
    gd = dims_of(Hqk, dk, Hv, dv)
    _check(lib().gdn_decode_fwd(*[_p(d) for d in D], ctypes.byref(gd), float(scale),
                                int(bool(use_qk_l2norm_in_kernel)), float(l2_eps), _p(desc(gate)),
                                _p(desc(norm_w)), float(rms_eps), _p(desc(out)), _stream(x_q)))
    return out


def _ws(nbytes: int, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def gdn_gated_norm_bwd(o, gate, weight, dout, eps: float = 1e-5, workspace=None):
    """Gradients of the gated norm. Returns (d_o, d_gate, d_weight F32)."""
    B, T, H, dv = o.shape
    d_o = torch.empty(o.shape, dtype=o.dtype, device=o.device)
    d_gate = torch.empty(gate.shape, dtype=gate.dtype, device=o.device)
    d_w = torch.empty(dv, dtype=torch.float32, device=o.device)
    nb = int(lib().gdn_gated_norm_bwd_workspace_bytes(B, T, H, dv))
    if workspace is None:
        workspace = _ws(nb, o.device)
    D = [desc(t) for t in (o, gate, weight)]
    E = [desc(t) for t in (dout, d_o, d_gate, d_w)]
    _check(lib().gdn_gated_norm_bwd(*[_p(d) for d in D], float(eps), *[_p(d) for d in E],
                                    ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
                                    _stream(o)))
    return d_o, d_gate, d_w


def gdn_prologue_bwd(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens, dims: Sequence[int],
                     d_qkv, d_g, d_beta, workspace=None):
    """Gradients of the prologue. Returns (dx_q, dx_k, dx_v, d_conv_w, d_conv_b or None,
    d_a, d_b, d_A_log, d_dt_bias)."""
    Hqk, dk, Hv, dv = dims
    B, T = x_q.shape[0], x_q.shape[1]
    C = 2 * Hqk * dk + Hv * dv
    dev, dt = x_q.device, x_q.dtype
    e = lambda *shape, d=dt: torch.empty(shape, dtype=d, device=dev)  # noqa: E731
    dxq, dxk, dxv = e(B, T, Hqk * dk), e(B, T, Hqk * dk), e(B, T, Hv * dv)
    dw = e(C, 4, d=torch.float32)
    dbias = e(C, d=torch.float32) if conv_b is not None else None
    da, db = e(B, T, Hv), e(B, T, Hv)
    dal, ddt = e(Hv, d=torch.float32), e(Hv, d=torch.float32)
    gd = dims_of(Hqk, dk, Hv, dv)
    nb = int(lib().gdn_prologue_bwd_workspace_bytes(B, T, ctypes.byref(gd)))
    if workspace is None:
        workspace = _ws(nb, dev)
    D = [desc(t) for t in (x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens)]
    E = [desc(t) for t in (d_qkv, d_g, d_beta, dxq, dxk, dxv, dw, dbias, da, db, dal, ddt)]
    _check(lib().gdn_prologue_bwd(*[_p(d) for d in D], ctypes.byref(gd), *[_p(d) for d in E],
                                  ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
                                  _stream(x_q)))
    return dxq, dxk, dxv, dw, dbias, da, db, dal, ddt


def gdn_chunk_rule_bwd_workspace_bytes(B: int, T: int, dims: Sequence[int], n_seqs: int = 0) -> int:
    gd = dims_of(*dims)
    return int(lib().gdn_chunk_rule_bwd_workspace_bytes(int(B), int(T), int(n_seqs), ctypes.byref(gd)))


def gdn_chunk_rule_bwd(q, k, v, g, beta, d_o, scale: float, use_qk_l2norm_in_kernel: bool = True,
                       l2_eps: float = 1e-6, cu_seqlens=None, initial_state=None, d_final_state=None,
                       want_d_initial_state: bool = False, grad_dtype=None, workspace=None):
    """Gradients of the chunked gated delta rule. Returns
    (dq, dk, dv, dg, dbeta, d_initial_state or None); dq, dk, dv in
    grad_dtype (default q's dtype), dg and dbeta FP32."""
    B, T, Hv, dv = v.shape
    Hqk, dk = q.shape[2], q.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.shape[0] - 1
    dev = q.device
    gdt = q.dtype if grad_dtype is None else grad_dtype
    e = lambda *shape, d=gdt: torch.empty(shape, dtype=d, device=dev)  # noqa: E731
    dq, dkk, dvv = e(B, T, Hqk, dk), e(B, T, Hqk, dk), e(B, T, Hv, dv)
    dg, db = e(B, T, Hv, d=torch.float32), e(B, T, Hv, d=torch.float32)
    dh0 = e(N, Hv, dv, dk, d=torch.float32) if want_d_initial_state else None
    if workspace is None:
        nb = gdn_chunk_rule_bwd_workspace_bytes(B, T, (Hqk, dk, Hv, dv), 0 if cu_seqlens is None else N)
        workspace = _ws(nb, dev)
    D = [desc(t) for t in (q, k, v, g, beta)]
    E = [desc(t) for t in (cu_seqlens, initial_state, d_o, d_final_state, dq, dkk, dvv, dg, db, dh0)]
    _check(lib().gdn_chunk_rule_bwd(*[_p(d) for d in D], float(scale), int(bool(use_qk_l2norm_in_kernel)),
                                    float(l2_eps), *[_p(d) for d in E], ctypes.c_void_p(workspace.data_ptr()),
                                    ctypes.c_size_t(workspace.numel()), _stream(q)))
    return dq, dkk, dvv, dg, db, dh0


def gdn_layer_bwd_workspace_bytes(B: int, T: int, dims: Sequence[int], dtype: torch.dtype,
                                  n_seqs: int = 0) -> int:
    gd = dims_of(*dims)
    return int(lib().gdn_layer_bwd_workspace_bytes(int(B), int(T), int(n_seqs), ctypes.byref(gd), DTYPE[dtype]))


def gdn_layer_bwd(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, cu_seqlens,
                  dims: Sequence[int], scale: float, d_out, use_qk_l2norm_in_kernel: bool = True,
                  l2_eps: float = 1e-6, rms_eps: float = 1e-5, workspace=None):
    """Gradients of gdn_layer_fwd. Returns (dx_q, dx_k, dx_v, d_conv_w, d_conv_b or None, d_a, d_b,
    d_A_log, d_dt_bias, d_gate, d_norm_w)."""
    return _layer_bwd(lib().gdn_layer_bwd, x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w,
                      cu_seqlens, dims, scale, d_out, use_qk_l2norm_in_kernel, l2_eps, rms_eps, workspace)


def _layer_bwd(fn, x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, cu_seqlens, dims, scale,
               d_out, use_qk_l2norm_in_kernel, l2_eps, rms_eps, workspace):
    Hqk, dk, Hv, dv = dims
    B, T = x_q.shape[0], x_q.shape[1]
    C = 2 * Hqk * dk + Hv * dv
    dev, dt = x_q.device, x_q.dtype
    e = lambda *shape, d=dt: torch.empty(shape, dtype=d, device=dev)  # noqa: E731
    dxq, dxk, dxv = e(B, T, Hqk * dk), e(B, T, Hqk * dk), e(B, T, Hv * dv)
    dw = e(C, 4, d=torch.float32)
    dbias = e(C, d=torch.float32) if conv_b is not None else None
    da, db = e(B, T, Hv), e(B, T, Hv)
    dal, ddt = e(Hv, d=torch.float32), e(Hv, d=torch.float32)
    dgate = e(B, T, Hv, dv, d=gate.dtype)
    dnw = e(dv, d=torch.float32)
    if workspace is None:
        n_seqs = 0 if cu_seqlens is None else cu_seqlens.shape[0] - 1
        workspace = _ws(gdn_layer_bwd_workspace_bytes(B, T, dims, dt, n_seqs), dev)
    gd = dims_of(Hqk, dk, Hv, dv)
    D = [desc(t) for t in (x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, cu_seqlens)]
    E = [desc(t) for t in (d_out, dxq, dxk, dxv, dw, dbias, da, db, dal, ddt, dgate, dnw)]
    _check(fn(*[_p(d) for d in D], ctypes.byref(gd), float(scale),
                               int(bool(use_qk_l2norm_in_kernel)), float(l2_eps), float(rms_eps),
                               *[_p(d) for d in E], ctypes.c_void_p(workspace.data_ptr()),
                               ctypes.c_size_t(workspace.numel()), _stream(x_q)))
    return dxq, dxk, dxv, dw, dbias, da, db, dal, ddt, dgate, dnw


def gdn_layer_bwd_saved(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, cu_seqlens,
                        dims: Sequence[int], scale: float, d_out, workspace, use_qk_l2norm_in_kernel: bool = True,
                        l2_eps: float = 1e-6, rms_eps: float = 1e-5):
    """gdn_layer_bwd from the activations a gdn_layer_fwd call with the same
    arguments left in `workspace` (gdn_layer_bwd_workspace_bytes bytes, given
    to that forward call). Returns what gdn_layer_bwd returns."""
    return _layer_bwd(lib().gdn_layer_bwd_saved, x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate,
                      norm_w, cu_seqlens, dims, scale, d_out, use_qk_l2norm_in_kernel, l2_eps, rms_eps, workspace)


def dtype_name(t: torch.dtype) -> str:
    return _NAMES[t]
