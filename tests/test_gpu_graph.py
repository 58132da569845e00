"""The library's calls inside a captured HIP graph: no allocation, no host
synchronisation and no memset nodes (every buffer, workspace included, is
the caller's), so a captured layer core or decode step replays with results
bitwise equal to the eager call. Each graph is replayed several times with
other eager work and synchronisations between replays, and every replay is
checked."""
import pytest
import torch

from linear_attention_rnn_qkv_amd import gdn, synth
from . import _gdn_helpers as H

pytestmark = pytest.mark.gpu


def _layer_case(cfg, over):
    s = synth.spec(cfg).replace(**over)
    x = H.to_dev(synth.make_inputs(s))
    dims = (s.Hqk, s.dk, s.Hv, s.dv)
    dt = synth.TORCH_DTYPE[s.act]
    n_seqs = 0 if x["cu_seqlens"] is None else x["cu_seqlens"].shape[0] - 1
    ws = torch.empty(gdn.gdn_layer_workspace_bytes(s.B, s.T, dims, dt, n_seqs), dtype=torch.uint8, device="cuda")
    out = torch.empty((s.B, s.T, s.Hv, s.dv), dtype=dt, device="cuda")

    def run():
        gdn.gdn_layer_fwd(x["x_q"], x["x_k"], x["x_v"], x["conv_w"], None, x["a"], x["b"], x["A_log"],
                          x["dt_bias"], x["gate"], x["norm_w"], x["cu_seqlens"], dims, s.dk ** -0.5, workspace=ws,
                          out=out)
    return run, out


@pytest.mark.parametrize("cfg,over", [(3, {"T": 200, "Hqk": 2, "Hv": 4}), (1, {"T": 130}),
                                      (4, {"lengths": (5, 70, 1, 64)}), (0, {"T": 100})],
                         ids=["bf16-two-kernel", "bf16-dk256-strided", "fp16-packed", "fp32-single-kernel"])
def test_layer_graph_replays_equal_eager(cfg, over):
    run, out = _layer_case(cfg, over)
    run()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
        run()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def test_decode_graph_replays_advance_the_state():
    """A captured decode step replayed T times equals T eager steps (the
    cache and state are updated in place by every replay)."""
    s = synth.spec(3).replace(B=8, T=6)
    x = H.to_dev(synth.make_inputs(s))
    dims = (s.Hqk, s.dk, s.Hv, s.dv)
    dt = synth.TORCH_DTYPE[s.act]
    tok = {k: x[k][:, 0].contiguous() for k in ("x_q", "x_k", "x_v", "a", "b", "gate")}

    def fresh():
        return (torch.zeros((s.B, 3, s.C), dtype=dt, device="cuda"),
                torch.zeros((s.B, s.Hv, s.dv, s.dk), dtype=torch.float32, device="cuda"),
                torch.empty((s.B, s.Hv, s.dv), dtype=dt, device="cuda"))

    def step(cache, state, out):
        gdn.gdn_decode_fwd(tok["x_q"], tok["x_k"], tok["x_v"], x["conv_w"], None, cache, tok["a"], tok["b"],
                           x["A_log"], x["dt_bias"], state, tok["gate"], x["norm_w"], dims, s.dk ** -0.5, out=out)

    ce, se, oe = fresh()
    eager = []
    for _ in range(4):
        step(ce, se, oe)
        eager.append(oe.clone())
    torch.cuda.synchronize()
    cg, sg, og = fresh()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(*fresh())  # warm-up on scratch buffers
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cg, sg, og)
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(og, eager[i]), f"replay {i}"
    assert torch.equal(sg, se) and torch.equal(cg, ce)


@pytest.mark.parametrize("cfg,over", [(2, {"T": 150, "Hqk": 1, "Hv": 2}), (4, {"lengths": (5, 70, 1, 64),
                                                                             "Hqk": 1, "Hv": 2}),
                                      (2, {"T": 200})],
                         ids=["bf16-gqa", "fp16-packed", "bf16-two-slice-state-passes"])
def test_layer_bwd_graph_replays_equal_eager(cfg, over):
    """The whole layer-core backward (its forward recomputed, then the three
    backward stages, every partial sum in the caller's workspace) captured
    once and replayed; every gradient of every replay equals the eager call."""
    s = synth.spec(cfg).replace(**over)
    x = H.to_dev(synth.make_inputs(s))
    dims = (s.Hqk, s.dk, s.Hv, s.dv)
    dt = synth.TORCH_DTYPE[s.act]
    n_seqs = 0 if x["cu_seqlens"] is None else x["cu_seqlens"].shape[0] - 1
    ws = torch.empty(gdn.gdn_layer_bwd_workspace_bytes(s.B, s.T, dims, dt, n_seqs), dtype=torch.uint8,
                     device="cuda")
    d_out = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 700 + cfg).cuda()

    def run():
        return gdn.gdn_layer_bwd(x["x_q"], x["x_k"], x["x_v"], x["conv_w"], None, x["a"], x["b"], x["A_log"],
                                 x["dt_bias"], x["gate"], x["norm_w"], x["cu_seqlens"], dims, s.dk ** -0.5, d_out,
                                 workspace=ws)

    eager = [t.clone() for t in run() if t is not None]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = [t for t in run() if t is not None]
    for i in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"replay {i}: gradient {j} differs from the eager call"
        run()  # eager work between replays
        torch.cuda.synchronize()


def test_layer_fwd_then_saved_bwd_graph_replays_equal_eager():
    """A training step of the layer core that keeps its activations:
    gdn_layer_fwd into the backward's workspace, then gdn_layer_bwd_saved on
    it, captured once and replayed; the output and every gradient of every
    replay equal the eager calls."""
    s = synth.spec(2).replace(T=150, Hqk=1, Hv=2)
    x = H.to_dev(synth.make_inputs(s))
    dims = (s.Hqk, s.dk, s.Hv, s.dv)
    dt = synth.TORCH_DTYPE[s.act]
    ws = torch.empty(gdn.gdn_layer_bwd_workspace_bytes(s.B, s.T, dims, dt, 0), dtype=torch.uint8, device="cuda")
    d_out = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 720).cuda()
    ins = (x["x_q"], x["x_k"], x["x_v"], x["conv_w"], None, x["a"], x["b"], x["A_log"], x["dt_bias"], x["gate"],
           x["norm_w"], None, dims, s.dk ** -0.5)

    def run():
        out = gdn.gdn_layer_fwd(*ins, workspace=ws)
        return [out] + [t for t in gdn.gdn_layer_bwd_saved(*ins, d_out, ws) if t is not None]

    eager = [t.clone() for t in run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    for i in range(3):
        for t in outs:
            t.zero_()
        ws.zero_()
        g.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"replay {i}: tensor {j} differs from the eager calls"
        run()  # eager work between replays
        torch.cuda.synchronize()
