"""GPU parity: every stage and the whole layer core, through the C ABI, against
the FP64 oracle on the same seeded inputs. Tolerance per output tensor:
max|gpu - oracle| <= tau * max|oracle|, tau = 1e-4 (FP32), 2e-2 (BF16/FP16).

Small cases span several 64-token chunks with a ragged tail; full-size cases
run the exact launch configuration the benchmark times and check sampled heads
(heads are independent, so the oracle of a head slice is exact for it).
Bitwise checks compare the kernels with themselves (GQA map vs replication,
strided vs contiguous gate, varlen vs separate calls, batch vs single rows,
run-to-run determinism).
"""
import math

import numpy as np
import pytest
import torch

from linear_attention_rnn_qkv_amd import gdn, synth
from oracle import gdn as O
from . import _gdn_helpers as H

pytestmark = pytest.mark.gpu

TAU = H.TAU
f64 = H.f64

SMALL = [
    ("tiny-fp32-T128", 0, {}),
    ("tiny-fp32-T100", 0, {"T": 100}),
    ("bf16-B2-hd256-T150-strided", 1, {"T": 150}),
    ("gqa-bf16-T300-fp32gate", 2, {"T": 300}),
    ("long-bf16-T200", 3, {"T": 200}),
    ("varlen-fp16-8seq", 4, {"lengths": (1, 63, 64, 65, 130, 2, 3, 200)}),
    # an odd GQA group (3 value heads per q/k head): the prep kernels then
    # take one value head per workgroup
    ("gqa3-bf16-T200", 3, {"T": 200, "Hqk": 2, "Hv": 6}),
]
IDS = [c[0] for c in SMALL]
# The recurrence runs as two kernels (chunk prep + chunk state) when given a
# workspace, as one kernel (chunk_rule_kernel) without; every recurrence test
# runs both.
PATHS = {"split": "auto", "one-kernel": None}


def _spec(cfg, over):
    return synth.spec(cfg).replace(**over)


def _dims(s):
    return (s.Hqk, s.dk, s.Hv, s.dv)


def _gpu_stage_inputs(s, qkv, g, beta, cu):
    dt = synth.TORCH_DTYPE[s.act]
    t = torch.from_numpy(qkv).to(dt).cuda()
    nq = s.Hqk * s.dk
    q = t[..., :nq].unflatten(-1, (s.Hqk, s.dk))
    k = t[..., nq:2 * nq].unflatten(-1, (s.Hqk, s.dk))
    v = t[..., 2 * nq:].unflatten(-1, (s.Hv, s.dv))
    gd = torch.from_numpy(g).float().cuda()
    bd = torch.from_numpy(beta).float().cuda()
    cud = None if cu is None else torch.from_numpy(cu.astype(np.int32)).cuda()
    return q, k, v, gd, bd, cud


# ---------------------------------------------------------------------------
# Prologue
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,cfg,over", SMALL, ids=IDS)
def test_prologue_parity(name, cfg, over):
    s = _spec(cfg, over)
    x = synth.make_inputs(s)
    xd = H.to_dev(x)
    qkv, g, beta = gdn.gdn_prologue_fwd(xd["x_q"], xd["x_k"], xd["x_v"], xd["conv_w"], None, xd["a"],
                                        xd["b"], xd["A_log"], xd["dt_bias"], xd["cu_seqlens"], _dims(s))
    torch.cuda.synchronize()
    rq, rg, rb = H.oracle_prologue(x, s)
    H.assert_close(f64(qkv), rq, TAU[s.act], "qkv")
    H.assert_close(f64(g), rg, 1e-5, "g")
    H.assert_close(f64(beta), rb, 1e-5, "beta")


# The prologue over every token of longer inputs against the oracle: 8192
# dense tokens (one 128-token tile per block and CU), 16383 and 33000 packed
# tokens (two and four blocks per CU, sequence boundaries inside tiles and a
# partial last tile).
DEEP = [
    ("gqa-bf16-T8192", 2, {}),
    ("varlen-fp16-16383-16seq", 4,
     {"lengths": (1, 700, 64, 65, 3000, 2, 129, 4096, 63, 2500, 1, 1500, 2000, 200, 1000, 1062)}),
    ("varlen-fp16-33000-9seq", 4,
     {"lengths": (5000, 1, 8191, 64, 12000, 3, 7000, 130, 611)}),
]


@pytest.mark.parametrize("name,cfg,over", DEEP, ids=[d[0] for d in DEEP])
def test_prologue_parity_launch_shapes(name, cfg, over):
    s = _spec(cfg, over)
    assert s.T == (8192 if cfg == 2 else sum(over["lengths"]))
    x = synth.make_inputs(s)
    xd = H.to_dev(x)
    qkv, g, beta = gdn.gdn_prologue_fwd(xd["x_q"], xd["x_k"], xd["x_v"], xd["conv_w"], None, xd["a"],
                                        xd["b"], xd["A_log"], xd["dt_bias"], xd["cu_seqlens"], _dims(s))
    torch.cuda.synchronize()
    rq, rg, rb = H.oracle_prologue(x, s)
    H.assert_close(f64(qkv), rq, TAU[s.act], "qkv")
    H.assert_close(f64(g), rg, 1e-5, "g")
    H.assert_close(f64(beta), rb, 1e-5, "beta")


@pytest.mark.parametrize("name,cfg,over", [SMALL[0], SMALL[2], SMALL[5]], ids=[IDS[0], IDS[2], IDS[5]])
def test_prologue_caller_side_l2norm(name, cfg, over):
    s = _spec(cfg, over)
    x = synth.make_inputs(s)
    xd = H.to_dev(x)
    qkv, _, _ = gdn.gdn_prologue_fwd(xd["x_q"], xd["x_k"], xd["x_v"], xd["conv_w"], None, xd["a"], xd["b"],
                                     xd["A_log"], xd["dt_bias"], xd["cu_seqlens"], _dims(s),
                                     caller_l2norm=True)
    torch.cuda.synchronize()
    xc = np.concatenate([f64(x["x_q"]), f64(x["x_k"]), f64(x["x_v"])], -1)
    y = O.causal_conv_silu(xc, f64(x["conv_w"]), None, H.cu_of(x))
    B, T, _ = y.shape
    nq = s.Hqk * s.dk
    y[..., :2 * nq] = O.l2norm(y[..., :2 * nq].reshape(B, T, 2 * s.Hqk, s.dk), 1e-6).reshape(B, T, 2 * nq)
    H.assert_close(f64(qkv), O.round_to(y, s.act), TAU[s.act], "qkv (caller-side L2)")


# ---------------------------------------------------------------------------
# Chunk rule
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name,cfg,over", SMALL, ids=IDS)
def test_chunk_rule_parity(name, cfg, over, path):
    s = _spec(cfg, over)
    x = synth.make_inputs(s)
    qkv, g, beta = H.oracle_prologue(x, s)
    q, k, v = H.split_qkv(qkv, s)
    cu = H.cu_of(x)
    qd, kd, vd, gd, bd, cud = _gpu_stage_inputs(s, qkv, g, beta, cu)
    for scale in (s.dk ** -0.5, 1.0):
        o, _ = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, scale, True, 1e-6, cud, workspace=PATHS[path])
        torch.cuda.synchronize()
        ro, _ = O.gated_delta_rule(q, k, v, g, beta, scale=scale, cu_seqlens=cu)
        H.assert_close(f64(o), O.round_to(ro, s.act), TAU[s.act], f"o (scale {scale:g})")


def _stress_inputs(cfg, over, seed, dt_bias=None):
    s = _spec(cfg, over)
    x = synth.make_inputs(s, dt_bias_override=dt_bias)
    qkv, g, beta = H.oracle_prologue(x, s)
    return s, x, qkv, g, beta


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("act_cfg", [0, 3])
def test_chunk_rule_state_in_out_slow_decay(act_cfg, path):
    # Stress set S1: dt_bias spread from -12 to 0 across heads, so some heads
    # keep their state for many chunks; a random initial state; final state out.
    over = {"T": 300, "Hqk": 2, "Hv": 4} if act_cfg == 3 else {"T": 200}
    s0 = _spec(act_cfg, over)
    s, x, qkv, g, beta = _stress_inputs(act_cfg, over, 0, synth.stress_dt_bias(s0.Hv))
    q, k, v = H.split_qkv(qkv, s)
    qd, kd, vd, gd, bd, _ = _gpu_stage_inputs(s, qkv, g, beta, None)
    S0 = synth.randn((s.B, s.Hv, s.dv, s.dk), "f32", 77).cuda() * 0.5
    scale = s.dk ** -0.5
    ws = PATHS[path]
    o, fin = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, scale, True, 1e-6, None, S0, output_final_state=True,
                                    workspace=ws)
    torch.cuda.synchronize()
    ro, rfin = O.gated_delta_rule(q, k, v, g, beta, scale=scale, initial_state=f64(S0), output_final_state=True)
    tau = TAU[s.act]
    H.assert_close(f64(o), O.round_to(ro, s.act), tau, "o")
    H.assert_close(f64(fin), rfin, tau, "final state")
    # state hand-off at a point inside a chunk equals one run
    cut = 137
    o1, f1 = gdn.gdn_chunk_rule_fwd(qd[:, :cut], kd[:, :cut], vd[:, :cut], gd[:, :cut], bd[:, :cut], scale, True,
                                    1e-6, None, S0, output_final_state=True, workspace=ws)
    o2, f2 = gdn.gdn_chunk_rule_fwd(qd[:, cut:], kd[:, cut:], vd[:, cut:], gd[:, cut:], bd[:, cut:], scale, True,
                                    1e-6, None, f1, output_final_state=True, workspace=ws)
    torch.cuda.synchronize()
    H.assert_close(f64(torch.cat([o1, o2], 1)), O.round_to(ro, s.act), tau, "o (hand-off)")
    H.assert_close(f64(f2), rfin, tau, "final state (hand-off)")


# The split path's state kernel has three forms: one 16-row value slice per
# workgroup, and 4 or 8 slices per workgroup sharing one copy of the k, q and
# record tiles, taken when the launch has at least 128 such workgroups
# (packed or batched sequences). These cases reach each multi-slice form
# (8 sequences x 32 heads at dv 128: 8 slices; 3 x 32 at dv 128 and
# 8 x 32 at dv 64: 4 slices; 8 batch rows: 8 slices over batch rows), with an
# initial state and the final state out, against the oracle and, bit for bit,
# against per-sequence calls, which run the one-slice kernel.
MULTI = [
    ("slices8-packed-fp16", 4, {"lengths": (1, 63, 64, 65, 130, 2, 3, 200)}),
    ("slices4-packed-fp16-3seq", 4, {"lengths": (100, 130, 64)}),
    ("slices4-packed-fp16-dv64", 4, {"lengths": (1, 63, 64, 65, 130, 2, 3, 200), "dv": 64}),
    ("slices8-batched-bf16-B8", 2, {"B": 8, "T": 100}),
]


@pytest.mark.parametrize("name,cfg,over", MULTI, ids=[m[0] for m in MULTI])
def test_chunk_rule_multi_slice_state_kernels(name, cfg, over):
    s, x, qkv, g, beta = _stress_inputs(cfg, over, 0)
    q, k, v = H.split_qkv(qkv, s)
    cu = H.cu_of(x)
    qd, kd, vd, gd, bd, cud = _gpu_stage_inputs(s, qkv, g, beta, cu)
    N = s.B if cu is None else len(cu) - 1
    S0 = synth.randn((N, s.Hv, s.dv, s.dk), "f32", 78).cuda() * 0.5
    scale = s.dk ** -0.5
    o, fin = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, scale, True, 1e-6, cud, S0, output_final_state=True)
    torch.cuda.synchronize()
    ro, rfin = O.gated_delta_rule(q, k, v, g, beta, scale=scale, cu_seqlens=cu, initial_state=f64(S0),
                                  output_final_state=True)
    tau = TAU[s.act]
    H.assert_close(f64(o), O.round_to(ro, s.act), tau, "o")
    H.assert_close(f64(fin), rfin, tau, "final state")
    for i in range(N):
        if cu is None:
            sl, rows = (slice(i, i + 1), slice(None)), slice(i, i + 1)
            oi, fi = gdn.gdn_chunk_rule_fwd(qd[sl], kd[sl], vd[sl], gd[sl], bd[sl], scale, True, 1e-6, None,
                                            S0[i:i + 1], output_final_state=True)
            torch.cuda.synchronize()
            assert torch.equal(oi, o[rows]), i
        else:
            a, b = int(cu[i]), int(cu[i + 1])
            oi, fi = gdn.gdn_chunk_rule_fwd(qd[:, a:b], kd[:, a:b], vd[:, a:b], gd[:, a:b], bd[:, a:b], scale, True,
                                            1e-6, None, S0[i:i + 1], output_final_state=True)
            torch.cuda.synchronize()
            assert torch.equal(oi, o[:, a:b]), i
        assert torch.equal(fi[0], fin[i]), i


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("cfg", [0, 3])
def test_chunk_rule_no_decay(cfg, path):
    # Stress set S2: g = 0 and beta ~ U(0, 1): nothing decays, so every chunk
    # boundary carries the full state.
    over = {"T": 260, "Hqk": 2, "Hv": 4} if cfg == 3 else {"T": 260}
    s, x, qkv, _, _ = _stress_inputs(cfg, over, 0)
    q, k, v = H.split_qkv(qkv, s)
    g = np.zeros((s.B, s.T, s.Hv))
    beta = O.round_to(synth.uniform((s.B, s.T, s.Hv), 0.0, 1.0, 5), "f32")
    qd, kd, vd, gd, bd, _ = _gpu_stage_inputs(s, qkv, g, beta, None)
    o, fin = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, 0.125, True, 1e-6, None, output_final_state=True,
                                    workspace=PATHS[path])
    torch.cuda.synchronize()
    ro, rfin = O.gated_delta_rule(q, k, v, g, beta, scale=0.125, output_final_state=True)
    H.assert_close(f64(o), O.round_to(ro, s.act), TAU[s.act], "o")
    H.assert_close(f64(fin), rfin, TAU[s.act], "final state")


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("dk,hqk,hv", [(64, 2, 8), (128, 4, 4), (64, 3, 3), (256, 2, 4), (256, 3, 3)],
                         ids=["dk64-G4", "dk128-G1", "dk64-G1", "dk256-G2", "dk256-G1"])
def test_chunk_rule_head_dims_and_group_sizes(dk, hqk, hv, path):
    # The two-kernel path has separate code for dk 64, 128 and 256 (its own
    # state kernel) and for odd and even GQA group sizes; each is checked
    # against the oracle with a state in and out.
    over = {"T": 300, "Hqk": hqk, "Hv": hv, "dk": dk}
    s, x, qkv, g, beta = _stress_inputs(3, over, 0)
    q, k, v = H.split_qkv(qkv, s)
    qd, kd, vd, gd, bd, _ = _gpu_stage_inputs(s, qkv, g, beta, None)
    S0 = synth.randn((s.B, s.Hv, s.dv, s.dk), "f32", 78).cuda() * 0.5
    scale = s.dk ** -0.5
    o, fin = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, scale, True, 1e-6, None, S0, output_final_state=True,
                                    workspace=PATHS[path])
    torch.cuda.synchronize()
    ro, rfin = O.gated_delta_rule(q, k, v, g, beta, scale=scale, initial_state=f64(S0), output_final_state=True)
    H.assert_close(f64(o), O.round_to(ro, s.act), TAU[s.act], "o")
    H.assert_close(f64(fin), rfin, TAU[s.act], "final state")


@pytest.mark.parametrize("path", list(PATHS))
def test_chunk_rule_empty_and_one_token_sequences(path):
    # Packed sequences of length 0 and 1 next to partial and full chunks: an
    # empty sequence hands its initial state through unchanged.
    s, x, qkv, g, beta = _stress_inputs(4, {"lengths": (0, 70, 0, 1, 64), "Hqk": 2, "Hv": 4}, 0)
    q, k, v = H.split_qkv(qkv, s)
    cu = H.cu_of(x)
    qd, kd, vd, gd, bd, cud = _gpu_stage_inputs(s, qkv, g, beta, cu)
    S0 = synth.randn((len(cu) - 1, s.Hv, s.dv, s.dk), "f32", 79).cuda() * 0.5
    o, fin = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, 0.1, True, 1e-6, cud, S0, output_final_state=True,
                                    workspace=PATHS[path])
    torch.cuda.synchronize()
    ro, rfin = O.gated_delta_rule(q, k, v, g, beta, scale=0.1, cu_seqlens=cu, initial_state=f64(S0),
                                  output_final_state=True)
    H.assert_close(f64(o), O.round_to(ro, s.act), TAU[s.act], "o")
    H.assert_close(f64(fin), rfin, TAU[s.act], "final state")
    assert torch.equal(fin[0], S0[0]) and torch.equal(fin[2], S0[2])


@pytest.mark.parametrize("path", list(PATHS))
def test_chunk_rule_dk256_packed_fp16_with_empty_sequences(path):
    # dk = 256 on packed FP16 sequences of length 0, 1, partial and several
    # chunks, with an initial state.
    s, x, qkv, g, beta = _stress_inputs(4, {"lengths": (0, 130, 1, 64, 0, 7), "Hqk": 2, "Hv": 4, "dk": 256,
                                            "dv": 64}, 0)
    q, k, v = H.split_qkv(qkv, s)
    cu = H.cu_of(x)
    qd, kd, vd, gd, bd, cud = _gpu_stage_inputs(s, qkv, g, beta, cu)
    S0 = synth.randn((len(cu) - 1, s.Hv, s.dv, s.dk), "f32", 81).cuda() * 0.5
    o, fin = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, 0.0625, True, 1e-6, cud, S0, output_final_state=True,
                                    workspace=PATHS[path])
    torch.cuda.synchronize()
    ro, rfin = O.gated_delta_rule(q, k, v, g, beta, scale=0.0625, cu_seqlens=cu, initial_state=f64(S0),
                                  output_final_state=True)
    H.assert_close(f64(o), O.round_to(ro, s.act), TAU[s.act], "o")
    H.assert_close(f64(fin), rfin, TAU[s.act], "final state")
    assert torch.equal(fin[0], S0[0]) and torch.equal(fin[4], S0[4])


def test_chunk_rule_dk256_narrow_dv_falls_back():
    # dk 256 with dv = 16 (not a multiple of the 32-row slices of the two-kernel
    # path) runs the single-kernel recurrence even with a workspace.
    s, x, qkv, g, beta = _stress_inputs(3, {"T": 100, "Hqk": 2, "Hv": 2, "dk": 256, "dv": 16}, 0)
    assert gdn.gdn_chunk_rule_workspace_bytes(s.B, s.T, (s.Hqk, s.dk, s.Hv, s.dv), torch.bfloat16) == 0
    q, k, v = H.split_qkv(qkv, s)
    qd, kd, vd, gd, bd, _ = _gpu_stage_inputs(s, qkv, g, beta, None)
    o, fin = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, 0.0625, True, 1e-6, output_final_state=True)
    torch.cuda.synchronize()
    ro, rfin = O.gated_delta_rule(q, k, v, g, beta, scale=0.0625, output_final_state=True)
    H.assert_close(f64(o), O.round_to(ro, s.act), TAU[s.act], "o")
    H.assert_close(f64(fin), rfin, TAU[s.act], "final state")


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("T", [1, 63, 65])
def test_chunk_rule_short_sequences(T, path):
    s, x, qkv, g, beta = _stress_inputs(3, {"T": T, "Hqk": 2, "Hv": 4}, 0)
    q, k, v = H.split_qkv(qkv, s)
    qd, kd, vd, gd, bd, _ = _gpu_stage_inputs(s, qkv, g, beta, None)
    o, fin = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, 0.1, True, 1e-6, output_final_state=True,
                                    workspace=PATHS[path])
    torch.cuda.synchronize()
    ro, rfin = O.gated_delta_rule(q, k, v, g, beta, scale=0.1, output_final_state=True)
    H.assert_close(f64(o), O.round_to(ro, s.act), TAU[s.act], "o")
    H.assert_close(f64(fin), rfin, TAU[s.act], "final state")


def test_chunk_rule_orthonormal_keys_retrieve_values():
    # Stress set S3 in FP32: g = 0, beta = 1 writes of orthonormal keys in the
    # first chunk, then beta = 0 reads in the second chunk with q = k_j must
    # return scale * v_j (the state crosses a chunk boundary unchanged).
    dk, dv, n = 64, 128, 64
    Qm, _ = np.linalg.qr(synth.uniform((dk, dk), -1, 1, 3))
    keys = Qm.T
    vals = synth.uniform((n, dv), -1, 1, 4)
    T = 2 * n
    k = np.zeros((1, T, 1, dk)); k[0, :n, 0] = keys; k[0, n:, 0] = keys
    q = np.zeros((1, T, 1, dk)); q[0, :n, 0] = keys; q[0, n:, 0] = keys[::-1]
    v = np.zeros((1, T, 1, dv)); v[0, :n, 0] = vals
    beta = np.zeros((1, T, 1)); beta[0, :n] = 1.0
    c = lambda a: torch.from_numpy(a).float().cuda()  # noqa: E731
    o, _ = gdn.gdn_chunk_rule_fwd(c(q), c(k), c(v), c(np.zeros((1, T, 1))), c(beta), 2.0, False, 1e-6)
    torch.cuda.synchronize()
    exp = np.concatenate([2.0 * vals, 2.0 * vals[::-1]])
    H.assert_close(f64(o)[0, :, 0], exp, 1e-4, "retrieved values")


@pytest.mark.parametrize("path", list(PATHS))
def test_chunk_rule_gqa_map_equals_replication_bitwise(path):
    s, x, qkv, g, beta = _stress_inputs(3, {"T": 150}, 0)
    qd, kd, vd, gd, bd, _ = _gpu_stage_inputs(s, qkv, g, beta, None)
    G = s.Hv // s.Hqk
    ws = PATHS[path]
    o1, _ = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, 0.1, True, 1e-6, workspace=ws)
    o2, _ = gdn.gdn_chunk_rule_fwd(qd.repeat_interleave(G, 2).contiguous(), kd.repeat_interleave(G, 2).contiguous(),
                                   vd, gd, bd, 0.1, True, 1e-6, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("path", list(PATHS))
def test_chunk_rule_deterministic_and_varlen_equals_separate_calls(path):
    s, x, qkv, g, beta = _stress_inputs(4, {"lengths": (5, 64, 100, 1, 77)}, 0)
    cu = H.cu_of(x)
    qd, kd, vd, gd, bd, cud = _gpu_stage_inputs(s, qkv, g, beta, cu)
    ws = PATHS[path]
    o1, f1 = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, 0.2, True, 1e-6, cud, output_final_state=True, workspace=ws)
    o2, f2 = gdn.gdn_chunk_rule_fwd(qd, kd, vd, gd, bd, 0.2, True, 1e-6, cud, output_final_state=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        oi, fi = gdn.gdn_chunk_rule_fwd(qd[:, a:b], kd[:, a:b], vd[:, a:b], gd[:, a:b], bd[:, a:b], 0.2, True, 1e-6,
                                        output_final_state=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(oi, o1[:, a:b]), i
        assert torch.equal(fi[0], f1[i]), i


def test_chunk_rule_in_kernel_l2_equals_caller_side():
    # Megatron-LM "fold q/k L2-norm into the gated_delta_rule kernel" (Why):
    # both routes normalise per head with eps 1e-6 and agree.
    s = _spec(2, {"T": 200})
    x = synth.make_inputs(s)
    xd = H.to_dev(x)
    args = (xd["x_q"], xd["x_k"], xd["x_v"], xd["conv_w"], None, xd["a"], xd["b"], xd["A_log"], xd["dt_bias"],
            None, _dims(s))
    nq = s.Hqk * s.dk

    def views(t):
        return (t[..., :nq].unflatten(-1, (s.Hqk, s.dk)), t[..., nq:2 * nq].unflatten(-1, (s.Hqk, s.dk)),
                t[..., 2 * nq:].unflatten(-1, (s.Hv, s.dv)))

    raw, g, beta = gdn.gdn_prologue_fwd(*args)
    nrm, _, _ = gdn.gdn_prologue_fwd(*args, caller_l2norm=True)
    o_in, _ = gdn.gdn_chunk_rule_fwd(*views(raw), g, beta, 0.1, True, 1e-6)
    o_caller, _ = gdn.gdn_chunk_rule_fwd(*views(nrm), g, beta, 0.1, False, 1e-6)
    torch.cuda.synchronize()
    H.assert_close(f64(o_caller), f64(o_in), TAU[s.act], "caller-side vs in-kernel")


# ---------------------------------------------------------------------------
# Gated norm
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,cfg,over", SMALL, ids=IDS)
def test_gated_norm_parity(name, cfg, over):
    s = _spec(cfg, over)
    x = synth.make_inputs(s)
    xd = H.to_dev(x)
    o = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 11).cuda()
    out = gdn.gdn_gated_norm_fwd(o, xd["gate"], xd["norm_w"], 1e-5)
    # strided recurrence output: o as a view with padding between heads
    o_pad = torch.zeros((s.B, s.T, s.Hv, s.dv + 8), dtype=o.dtype, device="cuda")
    o_pad[..., :s.dv] = o
    out2 = gdn.gdn_gated_norm_fwd(o_pad[..., :s.dv], xd["gate"], xd["norm_w"], 1e-5)
    torch.cuda.synchronize()
    ref = O.gated_rmsnorm(f64(o), f64(x["gate"]), f64(x["norm_w"]), 1e-5, s.act)
    H.assert_close(f64(out), ref, TAU[s.act], "out")
    assert torch.equal(out, out2)
    assert out.is_contiguous()


def test_gated_norm_strided_gate_equals_contiguous_bitwise():
    s = _spec(1, {"T": 64})
    x = H.to_dev(synth.make_inputs(s))
    assert not x["gate"].is_contiguous()
    o = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 12).cuda()
    a = gdn.gdn_gated_norm_fwd(o, x["gate"], x["norm_w"], 1e-5)
    b = gdn.gdn_gated_norm_fwd(o, x["gate"].contiguous(), x["norm_w"], 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    z = gdn.gdn_gated_norm_fwd(o, torch.zeros_like(x["gate"]), x["norm_w"], 1e-5)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z).item() == 0


# ---------------------------------------------------------------------------
# Layer
# ---------------------------------------------------------------------------
def _layer(xd, s, scale):
    return gdn.gdn_layer_fwd(xd["x_q"], xd["x_k"], xd["x_v"], xd["conv_w"], None, xd["a"], xd["b"], xd["A_log"],
                             xd["dt_bias"], xd["gate"], xd["norm_w"], xd["cu_seqlens"], _dims(s), scale)


@pytest.mark.parametrize("name,cfg,over", SMALL, ids=IDS)
def test_layer_parity(name, cfg, over):
    s = _spec(cfg, over)
    x = synth.make_inputs(s)
    xd = H.to_dev(x)
    scale = s.dk ** -0.5
    out = _layer(xd, s, scale)
    torch.cuda.synchronize()
    ref = H.oracle_layer(x, s, scale)
    H.assert_close(f64(out), ref, TAU[s.act], "layer out")


def test_layer_batch_rows_equal_single_row_calls_bitwise():
    s = _spec(1, {"T": 130})
    x = synth.make_inputs(s)
    xd = H.to_dev(x)
    out = _layer(xd, s, 0.0625)
    s1 = s.replace(B=1)
    for b in range(2):
        xb = {k: (v[b:b + 1] if k in ("x_q", "x_k", "x_v", "a", "b", "gate") else v) for k, v in xd.items()}
        ob = _layer(xb, s1, 0.0625)
        torch.cuda.synchronize()
        assert torch.equal(ob, out[b:b + 1]), b


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_layer_full_size_sampled_heads(cfg):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    runs on sampled query/key heads and the value heads that read them."""
    s = synth.spec(cfg)
    print(f"[full-size] workload {cfg} {s.name}: {s.tokens} tokens", flush=True)
    x = synth.make_inputs(s)
    xd = H.to_dev(x)
    scale = s.dk ** -0.5
    out = _layer(xd, s, scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    qk_heads = list(range(s.Hqk)) if cfg in (0, 1) else [0, s.Hqk - 1]
    xa, ss, vh = H.slice_heads(x, s, qk_heads)
    ref = H.oracle_layer_arrays(xa, ss, scale)
    rel = H.assert_close(f64(out[:, :, vh]), ref, TAU[s.act], f"layer out, workload {cfg}")
    print(f"[full-size] workload {cfg}: max rel err {rel:.3e}", flush=True)
