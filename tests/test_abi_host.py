"""Host-only tests of the C ABI: the library loads, exports every function the
header declares, sizes the workspace, and rejects invalid arguments from
metadata alone (no device work, so these run without a GPU). The descriptors
here point at host memory; every call is expected to fail validation before
anything is launched.
"""
import ctypes
import os
import re

import pytest
import torch

from linear_attention_rnn_qkv_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED = gdn.GDN_ERR_INVALID_VALUE, gdn.GDN_ERR_NOT_SUPPORTED


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    names = set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", hdr))
    assert names == {"gdn_last_error", "gdn_version", "gdn_prologue_fwd", "gdn_chunk_rule_fwd",
                     "gdn_chunk_rule_workspace_bytes", "gdn_gated_norm_fwd", "gdn_layer_workspace_bytes",
                     "gdn_layer_fwd", "gdn_decode_fwd", "gdn_gated_norm_bwd", "gdn_gated_norm_bwd_workspace_bytes",
                     "gdn_prologue_bwd", "gdn_prologue_bwd_workspace_bytes", "gdn_chunk_rule_bwd",
                     "gdn_chunk_rule_bwd_workspace_bytes", "gdn_layer_bwd", "gdn_layer_bwd_saved",
                     "gdn_layer_bwd_workspace_bytes",
                     "gdn_chunk_rule_fwd_noalloc"}
    L = gdn.lib()
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in gdn.gdn_version()


def test_workspace_bytes():
    def a256(x):
        return (x + 255) // 256 * 256
    B, T, dims = 2, 1000, (6, 256, 6, 512)
    C = 2 * 6 * 256 + 6 * 512
    expect = a256(B * T * C * 2) + 2 * a256(B * T * 6 * 4) + a256(B * T * 6 * 512 * 2)
    # dk = 256 BF16: chunk offsets, then one 14336-byte record per (chunk, value head)
    cws = a256((B + 1) * 4) + B * 16 * 6 * 14336
    assert gdn.gdn_chunk_rule_workspace_bytes(B, T, dims, torch.bfloat16) == cws
    assert gdn.gdn_layer_workspace_bytes(B, T, dims, torch.bfloat16) == expect + cws
    # FP32: the single-kernel recurrence, no chunk workspace
    assert gdn.gdn_chunk_rule_workspace_bytes(B, T, dims, torch.float32) == 0
    assert gdn.gdn_layer_workspace_bytes(B, T, (0, 64, 1, 64), torch.bfloat16) == 0
    # dk = 128 BF16: chunk offsets, then one 14336-byte record per (chunk, value head)
    d2 = (16, 128, 32, 128)
    rec = 14336
    assert gdn.gdn_chunk_rule_workspace_bytes(B, T, d2, torch.bfloat16) == a256((B + 1) * 4) + B * 16 * 32 * rec
    assert gdn.gdn_chunk_rule_workspace_bytes(1, T, d2, torch.float16, n_seqs=5) == a256(6 * 4) + (16 + 5) * 32 * rec
    assert gdn.gdn_chunk_rule_workspace_bytes(B, T, d2, torch.float32) == 0
    C2 = 2 * 16 * 128 + 32 * 128
    base = a256(B * T * C2 * 2) + 2 * a256(B * T * 32 * 4) + a256(B * T * 32 * 128 * 2)
    assert gdn.gdn_layer_workspace_bytes(B, T, d2, torch.bfloat16) == base + a256((B + 1) * 4) + B * 16 * 32 * rec


def _expect(status, fragment, fn, *args, **kw):
    with pytest.raises(gdn.GdnError) as e:
        fn(*args, **kw)
    assert e.value.status == status, str(e.value)
    assert fragment in str(e.value), str(e.value)


def _prologue_inputs(B=1, T=8, Hqk=2, dk=64, Hv=4, dv=64, dt=torch.bfloat16):
    nq, nv = Hqk * dk, Hv * dv
    C = 2 * nq + nv
    z = lambda *s, d=dt: torch.zeros(*s, dtype=d)  # noqa: E731
    return dict(x_q=z(B, T, nq), x_k=z(B, T, nq), x_v=z(B, T, nv), conv_w=z(C, 4), conv_b=None,
                a=z(B, T, Hv), b=z(B, T, Hv), A_log=z(Hv, d=torch.float32),
                dt_bias=z(Hv, d=torch.float32), cu_seqlens=None, dims=(Hqk, dk, Hv, dv))


def _pro(**over):
    kw = _prologue_inputs()
    kw.update(over)
    return gdn.gdn_prologue_fwd(**kw)


def test_prologue_rejections():
    x = _prologue_inputs()
    _expect(INVALID, "empty", gdn.gdn_prologue_fwd, **{**_prologue_inputs(T=0)})
    _expect(INVALID, "multiple of Hqk", _pro, dims=(3, 64, 4, 64))
    _expect(INVALID, "powers of two", _pro, dims=(2, 48, 4, 64))
    _expect(INVALID, "x_k: dtype", _pro, x_k=x["x_k"].half())
    _expect(INVALID, "innermost stride", _pro, x_q=torch.zeros(1, 8, 256, dtype=torch.bfloat16)[..., ::2])
    _expect(INVALID, "A_log: dtype", _pro, A_log=torch.zeros(4, dtype=torch.bfloat16))
    _expect(INVALID, "conv_w: dim 0", _pro, conv_w=torch.zeros(100, 4, dtype=torch.bfloat16))
    _expect(INVALID, "requires B == 1", gdn.gdn_prologue_fwd,
            **{**_prologue_inputs(B=2), "cu_seqlens": torch.tensor([0, 8], dtype=torch.int32)})
    _expect(INVALID, "cu_seqlens: dtype", _pro, cu_seqlens=torch.tensor([0, 8], dtype=torch.float32))
    C = 2 * 128 + 256
    qkv_nc = torch.zeros(1, 8, 2 * C, dtype=torch.bfloat16)[..., :C]
    _expect(INVALID, "out_qkv: must be contiguous", _pro, out_qkv=qkv_nc)
    buf = torch.zeros(1, 8, C, dtype=torch.bfloat16)
    _expect(INVALID, "overlaps", _pro, x_q=buf[..., :128], out_qkv=buf)
    _expect(INVALID, "descriptor is NULL", _pro, b=None)


def _chunk_inputs(B=1, T=8, Hqk=2, dk=64, Hv=4, dv=64, dt=torch.bfloat16):
    z = lambda *s, d=dt: torch.zeros(*s, dtype=d)  # noqa: E731
    return dict(q=z(B, T, Hqk, dk), k=z(B, T, Hqk, dk), v=z(B, T, Hv, dv),
                g=z(B, T, Hv, d=torch.float32), beta=z(B, T, Hv, d=torch.float32), scale=0.125)


def _chk(**over):
    kw = _chunk_inputs()
    kw.update(over)
    return gdn.gdn_chunk_rule_fwd(**kw)


def test_chunk_rule_rejections():
    _expect(INVALID, "empty", gdn.gdn_chunk_rule_fwd, **_chunk_inputs(T=0))
    _expect(UNSUPPORTED, "not instantiated", gdn.gdn_chunk_rule_fwd, **_chunk_inputs(dk=32))
    _expect(UNSUPPORTED, "not instantiated", gdn.gdn_chunk_rule_fwd, **_chunk_inputs(dk=256, dt=torch.float32))
    _expect(INVALID, "multiple of Hqk", gdn.gdn_chunk_rule_fwd, **_chunk_inputs(Hqk=3, Hv=4))
    _expect(INVALID, "initial_state: dim", _chk, initial_state=torch.zeros(1, 4, 64, 32))
    _expect(INVALID, "g: dtype", _chk, g=torch.zeros(1, 8, 4, dtype=torch.bfloat16))
    _expect(INVALID, "scale", _chk, scale=float("inf"))
    qbuf = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    _expect(INVALID, "out_o overlaps", _chk, q=qbuf, out_o=qbuf.view(1, 8, 1, 128)[..., :64]
            .expand(1, 8, 4, 64))
    raw = torch.zeros(1 * 8 * 2 * 64 + 1, dtype=torch.bfloat16)
    q_mis = raw[1:].view(1, 8, 2, 64)
    _expect(UNSUPPORTED, "16-byte aligned", _chk, q=q_mis)
    # chunk workspace: too small, misaligned, overlapping an argument
    n = gdn.gdn_chunk_rule_workspace_bytes(1, 8, (2, 64, 4, 64), torch.bfloat16)
    assert n > 0
    _expect(INVALID, "chunk workspace too small", _chk, workspace=torch.zeros(n - 256, dtype=torch.uint8))
    big = torch.zeros(n + 512, dtype=torch.uint8)
    off = (-big.data_ptr()) % 256
    _expect(INVALID, "256-byte aligned", _chk, workspace=big[off + 16: off + 16 + n])
    buf = torch.zeros(n + 4096, dtype=torch.uint8)
    off = (-buf.data_ptr()) % 256
    ws = buf[off: off + n]
    o_in_ws = ws[:8 * 4 * 64 * 2].view(torch.bfloat16).view(1, 8, 4, 64)
    _expect(INVALID, "workspace overlaps", _chk, workspace=ws, out_o=o_in_ws)


def _norm_inputs(B=1, T=4, H=2, dv=64, dt=torch.bfloat16, gdt=None, wdt=None):
    return dict(o=torch.zeros(B, T, H, dv, dtype=dt), gate=torch.zeros(B, T, H, dv, dtype=gdt or dt),
                weight=torch.ones(dv, dtype=wdt or dt))


def _nrm(**over):
    kw = _norm_inputs()
    kw.update(over)
    return gdn.gdn_gated_norm_fwd(**kw)


def test_gated_norm_rejections():
    # Megatron Core "GDN Elementwise Fusion", Post-GDR requirements: nonempty
    # output, matching gate shape, power-of-two head dim, gate in the
    # activation dtype or FP32, contiguous weight of length head_dim.
    _expect(INVALID, "empty", gdn.gdn_gated_norm_fwd, **_norm_inputs(T=0))
    _expect(INVALID, "power of two", gdn.gdn_gated_norm_fwd, **_norm_inputs(dv=96))
    _expect(UNSUPPORTED, "not instantiated", gdn.gdn_gated_norm_fwd, **_norm_inputs(dv=32))
    _expect(INVALID, "gate: dim", _nrm, gate=torch.zeros(1, 4, 3, 64, dtype=torch.bfloat16))
    _expect(INVALID, "gate: dtype", _nrm, gate=torch.zeros(1, 4, 2, 64, dtype=torch.float16))
    _expect(INVALID, "weight: must be contiguous", _nrm, weight=torch.ones(128, dtype=torch.bfloat16)[::2])
    _expect(INVALID, "weight: dim", _nrm, weight=torch.ones(32, dtype=torch.bfloat16))
    _expect(INVALID, "out: must be contiguous", _nrm,
            out=torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)[..., :64])
    _expect(INVALID, "out: dtype", _nrm, out=torch.zeros(1, 4, 2, 64, dtype=torch.float32))
    o = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    _expect(INVALID, "overlaps", _nrm, o=o, out=o)


def test_layer_rejections():
    x = _prologue_inputs()
    kw = dict(x, gate=torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16),
              norm_w=torch.ones(64, dtype=torch.bfloat16), scale=0.125)
    small = torch.zeros(256, dtype=torch.uint8)
    _expect(INVALID, "workspace too small", gdn.gdn_layer_fwd, **kw, workspace=small)
    n = gdn.gdn_layer_workspace_bytes(1, 8, (2, 64, 4, 64), torch.bfloat16)
    big = torch.zeros(n + 512, dtype=torch.uint8)
    off = (-big.data_ptr()) % 256
    mis = big[off + 8: off + 8 + n]
    _expect(INVALID, "256-byte aligned", gdn.gdn_layer_fwd, **kw, workspace=mis)


def _decode_inputs(N=3, Hqk=2, dk=64, Hv=4, dv=64, dt=torch.bfloat16):
    nq, nv = Hqk * dk, Hv * dv
    C = 2 * nq + nv
    z = lambda *s, d=dt: torch.zeros(*s, dtype=d)  # noqa: E731
    return dict(x_q=z(N, nq), x_k=z(N, nq), x_v=z(N, nv), conv_w=z(C, 4), conv_b=None,
                conv_state=z(N, 3, C), a=z(N, Hv), b=z(N, Hv), A_log=z(Hv, d=torch.float32),
                dt_bias=z(Hv, d=torch.float32), state=z(N, Hv, dv, dk, d=torch.float32),
                gate=z(N, Hv, dv), norm_w=z(dv), dims=(Hqk, dk, Hv, dv), scale=0.125)


def _dec(**over):
    kw = _decode_inputs()
    kw.update(over)
    return gdn.gdn_decode_fwd(**kw)


def test_decode_rejections():
    x = _decode_inputs()
    _expect(INVALID, "empty", gdn.gdn_decode_fwd, **_decode_inputs(N=0))
    _expect(INVALID, "multiple of Hqk", _dec, dims=(3, 64, 4, 64))
    _expect(UNSUPPORTED, "not instantiated", gdn.gdn_decode_fwd, **_decode_inputs(dk=32))
    _expect(UNSUPPORTED, "not instantiated", gdn.gdn_decode_fwd, **_decode_inputs(dv=32))
    _expect(UNSUPPORTED, "not instantiated", gdn.gdn_decode_fwd, **_decode_inputs(Hqk=1, Hv=128))
    _expect(INVALID, "conv_state: dim", _dec, conv_state=torch.zeros(3, 4, 512, dtype=torch.bfloat16))
    _expect(INVALID, "conv_state: dtype", _dec, conv_state=x["conv_state"].float())
    _expect(INVALID, "state: dtype", _dec, state=x["state"].bfloat16())
    _expect(INVALID, "state: must be contiguous", _dec,
            state=torch.zeros(3, 4, 64, 128, dtype=torch.float32)[..., :64])
    _expect(INVALID, "x_k: dtype", _dec, x_k=x["x_k"].half())
    _expect(INVALID, "gate: dtype", _dec, gate=x["gate"].half())
    _expect(INVALID, "out: must be contiguous", _dec,
            out=torch.zeros(3, 4, 128, dtype=torch.bfloat16)[..., :64])
    _expect(INVALID, "A_log: dtype", _dec, A_log=x["A_log"].bfloat16())
    _expect(INVALID, "l2_eps", _dec, l2_eps=float("nan"))
    _expect(INVALID, "overlaps", _dec, gate=x["gate"], out=x["gate"])
    buf = torch.zeros(3 * 3 * 512, dtype=torch.bfloat16)
    _expect(INVALID, "overlaps", _dec, conv_state=buf.view(3, 3, 512), x_v=buf[:768].view(3, 256))
    st = x["state"]
    _expect(INVALID, "must not overlap", _dec, state=st, conv_state=st.view(torch.bfloat16).view(-1)[:3 * 3 * 512]
            .view(3, 3, 512))
    big = torch.zeros(3 * 4 * 64 * 64 + 4, dtype=torch.float32)
    off = (-big.data_ptr() // 4) % 4
    _expect(UNSUPPORTED, "16-byte aligned", _dec, state=big[off + 1: off + 1 + 3 * 4 * 64 * 64].view(3, 4, 64, 64))


def test_error_message_is_per_call():
    with pytest.raises(gdn.GdnError):
        _nrm(o=torch.zeros(1, 0, 2, 64, dtype=torch.bfloat16))
    assert "empty" in gdn.gdn_last_error()


def test_backward_workspace_bytes_and_rejections():
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # gated norm: one [dv] FP32 partial per block, at most 8192 blocks of 4096 / dv rows
    assert gdn.lib().gdn_gated_norm_bwd_workspace_bytes(1, 100, 2, 128) == a256(7 * 128 * 4) + 32 * 128 * 4
    assert gdn.lib().gdn_gated_norm_bwd_workspace_bytes(1, 1 << 20, 32, 128) == 8192 * 128 * 4 + 32 * 128 * 4
    assert gdn.lib().gdn_gated_norm_bwd_workspace_bytes(1, 10, 2, 96) == 0
    # prologue: [token tiles][C][4] and [token tiles][C], [head tiles of 4096 / Hv tokens][Hv] twice,
    # then the reduction scratch [32][C * 4], all FP32. Tiles are 128 tokens, halved down to 32 while
    # the conv launch (one block per 1024 channels and tile) would have fewer than 2048 blocks: here
    # C = 512 gives one block per tile, so 600 tokens use 32-token tiles (19 of them)
    gd = gdn.dims_of(2, 64, 4, 64)
    C = 2 * 128 + 256
    assert gdn.lib().gdn_prologue_bwd_workspace_bytes(1, 600, gd) == (a256(19 * C * 16) + a256(19 * C * 4) +
                                                                      2 * a256(1 * 4 * 4) + a256(32 * C * 16))
    # 131072 tokens of the 16 -> 32 head geometry (C = 8192, 8 blocks per tile) keep 128-token tiles
    gd3 = gdn.dims_of(16, 128, 32, 128)
    assert gdn.lib().gdn_prologue_bwd_workspace_bytes(1, 131072, gd3) == (
        a256(1024 * 8192 * 16) + a256(1024 * 8192 * 4) + 2 * a256(1024 * 32 * 4) + a256(32 * 8192 * 16))
    o = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    w = torch.ones(64, dtype=torch.bfloat16)
    _expect(INVALID, "dout: dtype", gdn.gdn_gated_norm_bwd, o, o.clone(), w, o.half())
    _expect(INVALID, "workspace too small", gdn.gdn_gated_norm_bwd, o, o.clone(), w, o.clone(),
            workspace=torch.zeros(16, dtype=torch.uint8))
    x = _prologue_inputs()
    B, T, Hv = 1, 8, 4
    dq = torch.zeros(B, T, C, dtype=torch.bfloat16)
    dg, dbt = torch.zeros(B, T, Hv), torch.zeros(B, T, Hv)
    args = [x[k] for k in ("x_q", "x_k", "x_v", "conv_w", "conv_b", "a", "b", "A_log", "dt_bias", "cu_seqlens")]
    _expect(INVALID, "d_qkv: dim", gdn.gdn_prologue_bwd, *args, x["dims"], dq[..., :C - 8], dg, dbt)
    _expect(INVALID, "d_g: dtype", gdn.gdn_prologue_bwd, *args, x["dims"], dq, dg.bfloat16(), dbt)
    _expect(INVALID, "workspace too small", gdn.gdn_prologue_bwd, *args, x["dims"], dq, dg, dbt,
            workspace=torch.zeros(16, dtype=torch.uint8))


def _rule_bwd_inputs(B=1, T=8, Hqk=2, dk=64, Hv=4, dv=32, dt=torch.bfloat16):
    q, k = torch.zeros(B, T, Hqk, dk, dtype=dt), torch.zeros(B, T, Hqk, dk, dtype=dt)
    v, do = torch.zeros(B, T, Hv, dv, dtype=dt), torch.zeros(B, T, Hv, dv, dtype=dt)
    g, beta = torch.zeros(B, T, Hv), torch.zeros(B, T, Hv)
    return q, k, v, g, beta, do


def test_chunk_rule_bwd_workspace_bytes_and_rejections():
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # dense B=2, T=100: 4 chunk rows. Chunk offsets, unit q and k rows, their
    # inverse norms, gamma, (I + A)^-1 and P, S0 and dS, then R, Delta, dR',
    # then the 38912-byte records of the matrix-core state passes
    cb, Hqk, dk, Hv, dv = 4, 2, 64, 4, 32
    expect = (a256(3 * 4) + 2 * a256(cb * Hqk * 64 * dk * 4) + 2 * a256(cb * Hqk * 64 * 4) +
              a256(cb * Hv * 64 * 4) + 2 * a256(cb * Hv * 64 * 64 * 4) + 2 * a256(cb * Hv * dv * dk * 4) +
              3 * a256(cb * Hv * 64 * dv * 4) + a256(cb * Hv * 38912))
    assert gdn.gdn_chunk_rule_bwd_workspace_bytes(2, 100, (Hqk, dk, Hv, dv)) == expect
    # packed: ceil(T / 64) + n_seqs rows
    assert gdn.gdn_chunk_rule_bwd_workspace_bytes(1, 100, (1, 128, 1, 64), n_seqs=3) > 0
    assert gdn.gdn_chunk_rule_bwd_workspace_bytes(1, 100, (1, 256, 1, 64)) > 0
    assert gdn.gdn_chunk_rule_bwd_workspace_bytes(1, 100, (1, 512, 1, 64)) == 0  # dk 512 not built
    q, k, v, g, beta, do = _rule_bwd_inputs()
    _expect(INVALID, "d_o: dtype", gdn.gdn_chunk_rule_bwd, q, k, v, g, beta, do.half(), 0.125)
    _expect(INVALID, "dq: dtype", gdn.gdn_chunk_rule_bwd, q, k, v, g, beta, do, 0.125, grad_dtype=torch.float16)
    _expect(INVALID, "workspace too small", gdn.gdn_chunk_rule_bwd, q, k, v, g, beta, do, 0.125,
            workspace=torch.zeros(16, dtype=torch.uint8))
    _expect(INVALID, "d_final_state: dim", gdn.gdn_chunk_rule_bwd, q, k, v, g, beta, do, 0.125,
            d_final_state=torch.zeros(1, 4, 32, 32))
    q2, k2, v2, g2, b2, do2 = _rule_bwd_inputs(dk=512)
    _expect(UNSUPPORTED, "dk=512", gdn.gdn_chunk_rule_bwd, q2, k2, v2, g2, b2, do2, 0.0625)
    q3, k3, v3, g3, b3, do3 = _rule_bwd_inputs(dv=8)
    _expect(UNSUPPORTED, "dv=8", gdn.gdn_chunk_rule_bwd, q3, k3, v3, g3, b3, do3, 0.125)


def test_layer_bwd_workspace_bytes_and_rejections():
    # the layer backward holds the forward's stage outputs, the chunk forward's
    # workspace, d_o, d_qkv (act dtype), dg, dbeta and the three backward workspaces
    dims = (2, 64, 4, 64)
    n = gdn.gdn_layer_bwd_workspace_bytes(1, 100, dims, torch.bfloat16)
    assert n > gdn.gdn_chunk_rule_bwd_workspace_bytes(1, 100, dims) + 100 * (2 * 128 + 256) * 4
    assert gdn.gdn_layer_bwd_workspace_bytes(1, 100, (1, 512, 1, 64), torch.bfloat16) == 0
    x = _prologue_inputs()
    B, T, Hv, dv = 1, 8, 4, 64
    gate = torch.zeros(B, T, Hv, dv, dtype=torch.bfloat16)
    nw = torch.ones(dv, dtype=torch.bfloat16)
    d_out = torch.zeros(B, T, Hv, dv, dtype=torch.bfloat16)
    args = [x[k] for k in ("x_q", "x_k", "x_v", "conv_w", "conv_b", "a", "b", "A_log", "dt_bias")]
    _expect(INVALID, "workspace too small", gdn.gdn_layer_bwd, *args, gate, nw, x["cu_seqlens"], x["dims"], 0.125,
            d_out, workspace=torch.zeros(16, dtype=torch.uint8))
    nb = gdn.gdn_layer_bwd_workspace_bytes(B, T, x["dims"], torch.bfloat16)
    raw = torch.zeros(nb + 256, dtype=torch.uint8)
    off = (-raw.data_ptr()) % 256
    _expect(INVALID, "dout: dtype", gdn.gdn_layer_bwd, *args, gate, nw, x["cu_seqlens"], x["dims"], 0.125,
            d_out.half(), workspace=raw[off:off + nb])
    # the variant that reuses the forward's activations validates the same
    # way, and the forward's workspace layout is a prefix of the backward's
    _expect(INVALID, "workspace too small", gdn.gdn_layer_bwd_saved, *args, gate, nw, x["cu_seqlens"], x["dims"],
            0.125, d_out, torch.zeros(16, dtype=torch.uint8))
    _expect(INVALID, "dout: dtype", gdn.gdn_layer_bwd_saved, *args, gate, nw, x["cu_seqlens"], x["dims"], 0.125,
            d_out.half(), raw[off:off + nb])
    assert gdn.gdn_layer_workspace_bytes(B, T, x["dims"], torch.bfloat16) <= nb


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_binding_has_no_cpu_path():
    # every compute call goes through the library; the binding module imports
    # neither the oracle nor any fallback
    src = open(os.path.join(ROOT, "linear_attention_rnn_qkv_amd", "gdn.py")).read()
    assert "oracle" not in src and "numpy" not in src


def test_noalloc_rejects_inputs_beyond_the_static_scratch():
    # 80 chunks x 64 value heads of 14336-byte records exceed the 64 MiB
    # scratch: rejected from metadata before any device call
    T, Hqk, dk, Hv, dv = 80 * 64, 1, 64, 64, 16
    z = lambda *s, d=torch.bfloat16: torch.zeros(*s, dtype=d)  # noqa: E731
    need = gdn.gdn_chunk_rule_workspace_bytes(1, T, (Hqk, dk, Hv, dv), torch.bfloat16)
    assert need > gdn.GDN_NOALLOC_SCRATCH_BYTES
    _expect(INVALID, "static scratch", gdn.gdn_chunk_rule_fwd_noalloc, z(1, T, Hqk, dk), z(1, T, Hqk, dk),
            z(1, T, Hv, dv), z(1, T, Hv, d=torch.float32), z(1, T, Hv, d=torch.float32), 0.125,
            out_o=z(1, T, Hv, dv))
    # and the ordinary validation runs first
    _expect(INVALID, "powers of two", gdn.gdn_chunk_rule_fwd_noalloc, z(1, T, Hqk, dk + 1), z(1, T, Hqk, dk),
            z(1, T, Hv, dv), z(1, T, Hv, d=torch.float32), z(1, T, Hv, d=torch.float32), 0.125,
            out_o=z(1, T, Hv, dv))


def test_prologue_bwd_token_tile_per_size():
    """The prologue backward's token tile (128 tokens, halved down to 32 while
    its conv launch would have fewer than 2048 blocks) read back from the
    workspace it asks for: per tile, [C][4] and [C] FP32 partial sums."""
    def a256(x):
        return (x + 255) // 256 * 256
    dims = (16, 128, 32, 128)
    C = 2 * 16 * 128 + 32 * 128

    def expect(T, tile):
        nt = (T + tile - 1) // tile
        head_tile = 4096 // 32
        nh = (T + head_tile - 1) // head_tile
        return a256(nt * C * 16) + a256(nt * C * 4) + 2 * a256(nh * 32 * 4) + a256(32 * C * 16)
    for T, tile in [(8192, 32), (16384, 64), (32768, 128), (65536, 128), (131072, 128), (100, 32)]:
        got = gdn.lib().gdn_prologue_bwd_workspace_bytes(1, T, ctypes.byref(gdn.dims_of(*dims)))
        assert got == expect(T, tile), (T, tile, got)
