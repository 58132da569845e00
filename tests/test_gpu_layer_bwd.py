"""GPU parity of gdn_layer_bwd (through the C ABI): the gradients of the whole
layer core against the FP64 oracle's stage backwards chained at the stored
forward values (the oracle's own conv output, g, beta and recurrence output,
rounded where the layer materialises them; d_o rounded to the activation
dtype as the layer stores it). Tolerance per output tensor: max|gpu -
oracle| <= tau * max|oracle|, tau = 1e-4 (FP32 workloads) and, for 16-bit
workloads, 2e-2: the stage inputs on the two sides are stored forward values
that agree to the forward's bar, not bit for bit."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_qkv_amd import gdn, synth
from oracle import backward as OB
from oracle import gdn as O
from . import _gdn_helpers as H

pytestmark = pytest.mark.gpu

TAU = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
f64 = H.f64

CASES = [
    ("fp32-gqa-T100-bias", 0, {"T": 100, "Hqk": 2, "Hv": 4, "dv": 64}, True),
    ("bf16-gqa-fp32gate-T150", 2, {"T": 150, "Hqk": 1, "Hv": 2}, False),
    ("fp16-packed-with-empty", 4, {"lengths": (1, 63, 0, 65, 130), "Hqk": 1, "Hv": 2}, False),
    ("bf16-hd256-strided-T70", 1, {"T": 70, "B": 1, "Hqk": 1, "Hv": 1}, False),
]


@pytest.mark.parametrize("name,cfg,over,bias", CASES, ids=[c[0] for c in CASES])
def test_layer_bwd_parity(name, cfg, over, bias):
    s = synth.spec(cfg).replace(**over)
    x = H.to_dev(synth.make_inputs(s))
    if bias:
        x["conv_b"] = (0.1 * synth.randn((s.C,), "f32", 56)).cuda()
    dims = (s.Hqk, s.dk, s.Hv, s.dv)
    scale = s.dk ** -0.5
    d_out = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 600 + cfg).cuda()
    args = (x["x_q"], x["x_k"], x["x_v"], x["conv_w"], x["conv_b"], x["a"], x["b"], x["A_log"], x["dt_bias"],
            x["gate"], x["norm_w"], x["cu_seqlens"], dims, scale, d_out)
    got = gdn.gdn_layer_bwd(*args)
    again = gdn.gdn_layer_bwd(*args)
    torch.cuda.synchronize()

    cu = H.cu_of(x)
    _, st = O.layer(f64(x["x_q"]), f64(x["x_k"]), f64(x["x_v"]), f64(x["conv_w"]), f64(x["conv_b"]),
                    f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]), f64(x["gate"]),
                    f64(x["norm_w"]), Hqk=s.Hqk, dk=s.dk, Hv=s.Hv, dv=s.dv, act=s.act, scale=scale,
                    cu_seqlens=cu, return_stages=True)
    q, k, v = H.split_qkv(st["qkv"], s)
    r_do, r_dgate, r_dw = OB.gated_rmsnorm_bwd(st["o"], f64(x["gate"]), f64(x["norm_w"]), f64(d_out), 1e-5)
    d_o = O.round_to(r_do, s.act)
    dq, dk, dv, dg, db, _ = OB.chunk_rule_bwd(q, k, v, st["g"], st["beta"], d_o, scale, True, 1e-6, cu)
    B, T = s.B, s.T
    dqkv = np.concatenate([dq.reshape(B, T, -1), dk.reshape(B, T, -1), dv.reshape(B, T, -1)], -1)
    pro = OB.prologue_bwd(f64(x["x_q"]), f64(x["x_k"]), f64(x["x_v"]), f64(x["conv_w"]), f64(x["conv_b"]),
                          f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]), dqkv, dg, db, cu)
    names = ("dx_q", "dx_k", "dx_v", "d_conv_w", "d_conv_b", "d_a", "d_b", "d_A_log", "d_dt_bias", "d_gate",
             "d_norm_w")
    refs = list(pro) + [r_dgate, r_dw]
    tau = TAU[s.act]
    for n, g_, r in zip(names, got, refs):
        if r is None:
            assert g_ is None, n
            continue
        H.assert_close(f64(g_), r, tau, n)
    for n, a_, b_ in zip(names, got, again):
        if a_ is not None:
            assert torch.equal(a_, b_), f"{n} differs between calls"


@pytest.mark.parametrize("name,cfg,over,bias", CASES, ids=[c[0] for c in CASES])
def test_layer_bwd_saved_equals_recomputed(name, cfg, over, bias):
    """gdn_layer_bwd_saved after a gdn_layer_fwd into the same workspace gives
    gdn_layer_bwd's outputs bit for bit (the forward's qkv, g, beta and o are
    what the recompute would write; the kernels are deterministic)."""
    s = synth.spec(cfg).replace(**over)
    x = H.to_dev(synth.make_inputs(s))
    if bias:
        x["conv_b"] = (0.1 * synth.randn((s.C,), "f32", 56)).cuda()
    dims = (s.Hqk, s.dk, s.Hv, s.dv)
    scale = s.dk ** -0.5
    d_out = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 610 + cfg).cuda()
    ins = (x["x_q"], x["x_k"], x["x_v"], x["conv_w"], x["conv_b"], x["a"], x["b"], x["A_log"], x["dt_bias"],
           x["gate"], x["norm_w"], x["cu_seqlens"], dims, scale)
    n_seqs = 0 if x["cu_seqlens"] is None else x["cu_seqlens"].shape[0] - 1
    nb = gdn.gdn_layer_bwd_workspace_bytes(s.B, s.T, dims, x["x_q"].dtype, n_seqs)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = gdn.gdn_layer_fwd(*ins, workspace=ws)
    saved = gdn.gdn_layer_bwd_saved(*ins, d_out, ws)
    ref_out = gdn.gdn_layer_fwd(*ins)
    ref = gdn.gdn_layer_bwd(*ins, d_out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    names = ("dx_q", "dx_k", "dx_v", "d_conv_w", "d_conv_b", "d_a", "d_b", "d_A_log", "d_dt_bias", "d_gate",
             "d_norm_w")
    for n, a_, b_ in zip(names, saved, ref):
        if b_ is None:
            assert a_ is None, n
        else:
            assert torch.equal(a_, b_), f"{n} differs from the recomputing backward"
