"""GPU parity of gdn_chunk_rule_bwd (through the C ABI) against the FP64
oracle (float64 autograd of the token-by-token gated delta rule) on the same
seeded inputs. Tolerance per output tensor: max|gpu - oracle| <= tau *
max|oracle|, tau = 1e-4 (FP32 workloads), 5e-3 (BF16/FP16). Gradients are
also checked to be identical across two calls (no atomics)."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_qkv_amd import gdn, synth
from oracle import backward as OB
from oracle import gdn as O
from . import _gdn_helpers as H

pytestmark = pytest.mark.gpu

# Gradient bar for 16-bit workloads: 5e-3 of the largest reference gradient,
# the bar the fused-conv pull request's test plan holds parameter gradients
# to; FP32 workloads keep 1e-4.
TAU = {"f32": 1e-4, "bf16": 5e-3, "f16": 5e-3}
f64 = H.f64
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def _inputs(cfg, over):
    s = synth.spec(cfg).replace(**over)
    x = synth.make_inputs(s)
    qkv, g, beta = H.oracle_prologue(x, s)
    q, k, v = H.split_qkv(qkv, s)
    return s, q, k, v, g, beta, H.cu_of(x)


def _dev(s, arrs, cu):
    dt = synth.TORCH_DTYPE[s.act]
    q, k, v, g, beta = arrs
    out = [torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda() for a in (q, k, v)]
    out += [torch.from_numpy(np.ascontiguousarray(a)).float().cuda() for a in (g, beta)]
    cud = None if cu is None else torch.from_numpy(cu.astype(np.int32)).cuda()
    return out, cud


def _check(got, ref, tau):
    for n, a, r in zip(NAMES, got, ref):
        if r is None:
            assert a is None, n
            continue
        H.assert_close(f64(a), r, tau, n)


CASES = [
    # name, workload, overrides, initial state and final-state gradient, L2 fold
    ("fp32-gqa-T100-state", 0, {"T": 100, "Hqk": 2, "Hv": 4, "dv": 64, "B": 2}, True, True),
    ("bf16-dk128-T150", 2, {"T": 150, "Hqk": 1, "Hv": 2}, False, True),
    ("fp16-packed-with-empty", 4, {"lengths": (1, 63, 0, 64, 65, 2, 0, 130), "Hqk": 1, "Hv": 2}, True, True),
    ("bf16-dk64-dv256-T200", 0, {"act": "bf16", "T": 200, "Hqk": 1, "Hv": 1, "dv": 256}, True, True),
    ("fp32-no-l2-T90", 0, {"T": 90, "Hqk": 1, "Hv": 2, "dv": 64}, False, False),
    ("bf16-group4-T129", 2, {"T": 129, "Hqk": 2, "Hv": 8, "dv": 64}, True, True),
    ("fp16-group3-T150", 4, {"T": 150, "lengths": None, "Hqk": 2, "Hv": 6, "dv": 64}, True, True),
    ("bf16-dk256-dv512-T130", 1, {"T": 130, "B": 1, "Hqk": 1, "Hv": 1}, True, True),
    ("fp32-dk256-gqa-T70", 0, {"T": 70, "dk": 256, "dv": 64, "Hqk": 1, "Hv": 2}, True, True),
]


@pytest.mark.parametrize("name,cfg,over,state,use_l2", CASES, ids=[c[0] for c in CASES])
def test_chunk_rule_bwd_parity(name, cfg, over, state, use_l2):
    s, q, k, v, g, beta, cu = _inputs(cfg, over)
    if not use_l2:  # rows of norm 0.9 so that the unnormalised recurrence stays bounded
        q = O.round_to(0.9 * O.l2norm(q), s.act)
        k = O.round_to(0.9 * O.l2norm(k), s.act)
    (qd, kd, vd, gd, bd), cud = _dev(s, (q, k, v, g, beta), cu)
    N = s.n_seqs
    h0 = synth.randn((N, s.Hv, s.dv, s.dk), "f32", 400 + cfg).cuda() * 0.5 if state else None
    dht = synth.randn((N, s.Hv, s.dv, s.dk), "f32", 410 + cfg).cuda() * 0.1 if state else None
    do = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 420 + cfg).cuda()
    scale = s.dk ** -0.5
    args = (qd, kd, vd, gd, bd, do, scale, use_l2, 1e-6, cud, h0, dht)
    got = gdn.gdn_chunk_rule_bwd(*args, want_d_initial_state=state)
    again = gdn.gdn_chunk_rule_bwd(*args, want_d_initial_state=state)
    torch.cuda.synchronize()
    ref = OB.chunk_rule_bwd(q, k, v, g, beta, f64(do), scale, use_l2, 1e-6, cu,
                            None if h0 is None else f64(h0), None if dht is None else f64(dht))
    _check(got, ref, TAU[s.act])
    for n, a, b in zip(NAMES, got, again):
        if a is not None:
            assert torch.equal(a, b), f"{n} differs between calls"


def test_chunk_rule_bwd_f32_gradients_of_bf16_inputs():
    s, q, k, v, g, beta, cu = _inputs(2, {"T": 130, "Hqk": 2, "Hv": 4})
    (qd, kd, vd, gd, bd), cud = _dev(s, (q, k, v, g, beta), cu)
    do = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 430).cuda()
    got = gdn.gdn_chunk_rule_bwd(qd, kd, vd, gd, bd, do, 0.1, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert all(t.dtype == torch.float32 for t in got[:3])
    ref = OB.chunk_rule_bwd(q, k, v, g, beta, f64(do), 0.1)
    # FP32 outputs from exact 16-bit inputs: only FP32 arithmetic separates them
    _check(got, ref, 1e-4)


def test_chunk_rule_bwd_strided_views_equal_contiguous():
    # q, k, v as channel views of one [B, T, C] buffer and d_o with a padded
    # row pitch give the same bits as contiguous copies
    s, q, k, v, g, beta, cu = _inputs(2, {"T": 100, "Hqk": 2, "Hv": 4})
    dt = synth.TORCH_DTYPE[s.act]
    nq = s.Hqk * s.dk
    qkv = torch.from_numpy(np.concatenate([q.reshape(1, s.T, -1), k.reshape(1, s.T, -1), v.reshape(1, s.T, -1)],
                                          -1)).to(dt).cuda()
    qv = qkv[..., :nq].unflatten(-1, (s.Hqk, s.dk))
    kv = qkv[..., nq:2 * nq].unflatten(-1, (s.Hqk, s.dk))
    vv = qkv[..., 2 * nq:].unflatten(-1, (s.Hv, s.dv))
    gd = torch.from_numpy(g).float().cuda()
    bd = torch.from_numpy(beta).float().cuda()
    pad = synth.randn((s.B, s.T, s.Hv, s.dv + 16), s.act, 440).cuda()
    do = pad[..., :s.dv]
    a = gdn.gdn_chunk_rule_bwd(qv, kv, vv, gd, bd, do, 0.09)
    b = gdn.gdn_chunk_rule_bwd(qv.contiguous(), kv.contiguous(), vv.contiguous(), gd, bd, do.contiguous(), 0.09)
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, a, b):
        if x is not None:
            assert torch.equal(x, y), n


# 16-bit workloads (BF16 and FP16) run matrix-core kernels where their
# operand rows allow: the two state passes need 16-byte q, k, v and d_o rows,
# the gradient kernel dv a multiple of 32 and 8-byte d_o and v rows. These cases
# pick each mix, in both 16-bit types.
MIXES = [
    # name, dv, d_o row pitch (elements past dv)
    ("states-mma-grad-fp32-dv16", 16, 0),
    ("states-fp32-grad-mma-do8", 64, 4),
    ("all-fp32-do2", 64, 1),
]


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("name,dv,pad", MIXES, ids=[m[0] for m in MIXES])
def test_chunk_rule_bwd_kernel_mixes(name, dv, pad, act):
    s, q, k, v, g, beta, cu = _inputs(2, {"act": act, "T": 130, "Hqk": 1, "Hv": 2, "dk": 64, "dv": dv, "B": 1})
    (qd, kd, vd, gd, bd), cud = _dev(s, (q, k, v, g, beta), cu)
    buf = synth.randn((s.B, s.T, s.Hv, dv + pad), s.act, 450).cuda()
    do = buf[..., :dv]
    h0 = synth.randn((1, s.Hv, dv, s.dk), "f32", 451).cuda() * 0.5
    dht = synth.randn((1, s.Hv, dv, s.dk), "f32", 452).cuda() * 0.1
    got = gdn.gdn_chunk_rule_bwd(qd, kd, vd, gd, bd, do, 0.125, True, 1e-6, None, h0, dht, want_d_initial_state=True)
    torch.cuda.synchronize()
    ref = OB.chunk_rule_bwd(q, k, v, g, beta, f64(do), 0.125, True, 1e-6, None, f64(h0), f64(dht))
    _check(got, ref, TAU[act])


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("where", ["tail", "mid"])
def test_chunk_rule_bwd_full_size_window(where, act):
    """The 131072-token workload's shape (16 q/k heads, 32 value heads, dk = dv
    = 128; BF16, and the same shape in FP16) in one call, with d_o zero except
    on a window of 150 tokens:
    the sequence's last 150 tokens, or 150 tokens from 70037 (not a multiple
    of the 64-token chunk). Every token of every head is checked:
      * tokens [start - 100, end): all five gradients against the oracle
        (float64 autograd of the token recurrence over [start - 356, end),
        all heads, from a zero state; the state dropped at start - 356 reaches
        the compared tokens scaled by at most exp(sum of g over 256 tokens),
        asserted below 1e-12);
      * dq is exactly zero outside the window (o_t depends on q_t only);
      * after the window every gradient is exactly zero (no later d_o);
      * before start - 100 every gradient is below the carried-decay bound:
        it reaches token t through the state, scaled by
        exp(sum of g over [t + 1, start)) <= D_h = exp(sum over the 100 tokens
        before start), so |grad| <= 1e4 * D_h * (largest gradient).
    Inputs are seeded draws (q, k, v ~ N(0, 1); g ~ -U(0.01, 0.5);
    beta ~ U(0.05, 1))."""
    s = synth.spec(3)
    B, T, Hqk, dk, Hv, dv = s.B, s.T, s.Hqk, s.dk, s.Hv, s.dv
    print(f"[bwd full size] window {where} {act}", flush=True)
    q = synth.randn((B, T, Hqk, dk), act, 500)
    k = synth.randn((B, T, Hqk, dk), act, 501)
    v = synth.randn((B, T, Hv, dv), act, 502)
    g = O.round_to(-synth.uniform((B, T, Hv), 0.01, 0.5, 503), "f32")
    beta = O.round_to(synth.uniform((B, T, Hv), 0.05, 1.0, 504), "f32")
    W, W1, LEAD = 150, 100, 256
    start = T - W if where == "tail" else 70037
    end = start + W
    assert where == "tail" or start % 64 != 0
    t1, t0 = start - W1, start - W1 - LEAD
    do = torch.zeros((B, T, Hv, dv), dtype=synth.TORCH_DTYPE[act])
    do[:, start:end] = synth.randn((B, W, Hv, dv), act, 505)
    scale = dk ** -0.5
    got = gdn.gdn_chunk_rule_bwd(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(g).float().cuda(),
                                 torch.from_numpy(beta).float().cuda(), do.cuda(), scale)
    torch.cuda.synchronize()
    dq, dkk, dvv, dg, db, _ = got
    for n, x in zip(NAMES, got[:5]):
        assert torch.isfinite(x).all(), n
    # exact zeros
    assert not dq[:, :start].any() and not dq[:, end:].any(), "dq outside the window"
    for n, x in zip(NAMES[:5], (dq, dkk, dvv, dg, db)):
        assert not x[:, end:].any(), f"{n} after the window"
    # the oracle over [t0, end), every head
    lead = np.exp(np.sum(g[0, t0:t1], axis=0))
    assert float(lead.max()) < 1e-12, lead.max()
    ref = OB.chunk_rule_bwd(f64(q[:, t0:end]), f64(k[:, t0:end]), f64(v[:, t0:end]), g[:, t0:end],
                            beta[:, t0:end], f64(do[:, t0:end]), scale)
    tau = TAU[act]
    w = slice(t1 - t0, end - t0)
    for n, x, r in zip(NAMES, (dq, dkk, dvv, dg, db), ref[:5]):
        H.assert_close(f64(x[:, t1:end]), r[:, w], tau, n)
    # the carried part alone (tokens before the window), against its own scale
    for n, x, r in ((NAMES[1], dkk, ref[1]), (NAMES[2], dvv, ref[2])):
        H.assert_close(f64(x[:, t1:start]), r[:, w][:, :W1], tau, f"{n} before the window")
    assert float(np.abs(ref[2][:, w][:, :W1]).max()) > 0
    # carried-decay bound before t1
    D = np.exp(np.sum(g[0, t1:start], axis=0))  # [Hv]
    bound = 1e4 * float(D.max())
    assert bound < 1e-3, bound
    for n, x, r in zip(NAMES[1:5], (dkk, dvv, dg, db), ref[1:5]):
        big = float(np.abs(r[:, w]).max())
        before = x[:, :t1].float().abs()
        worst = float(before.max()) if before.numel() else 0.0
        assert worst <= bound * big, (n, worst, bound * big)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_chunk_rule_bwd_slow_decay(act):
    """Slow decay (g ~ -U(1e-4, 2e-3), the state carried across 2048 tokens
    with little loss) at dk = dv = 128, one q/k head and its two value heads,
    a random initial state and a final-state gradient: the matrix-core
    passes carry the states and their gradients as split 16-bit operands, and
    this is where they grow largest; FP16 halves have the narrower range.
    Every gradient against the oracle at the 16-bit bar."""
    B, T, Hqk, dk, Hv, dv = 1, 2048, 1, 128, 2, 128
    q = synth.randn((B, T, Hqk, dk), act, 520)
    k = synth.randn((B, T, Hqk, dk), act, 521)
    v = synth.randn((B, T, Hv, dv), act, 522)
    g = O.round_to(-synth.uniform((B, T, Hv), 1e-4, 2e-3, 523), "f32")
    beta = O.round_to(synth.uniform((B, T, Hv), 0.05, 1.0, 524), "f32")
    do = synth.randn((B, T, Hv, dv), act, 525)
    h0 = synth.randn((1, Hv, dv, dk), "f32", 526)
    dht = synth.randn((1, Hv, dv, dk), "f32", 527)
    scale = dk ** -0.5
    got = gdn.gdn_chunk_rule_bwd(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(g).float().cuda(),
                                 torch.from_numpy(beta).float().cuda(), do.cuda(), scale, True, 1e-6, None,
                                 h0.cuda(), dht.cuda(), want_d_initial_state=True)
    torch.cuda.synchronize()
    ref = OB.chunk_rule_bwd(f64(q), f64(k), f64(v), g, beta, f64(do), scale, True, 1e-6, None, f64(h0), f64(dht))
    _check(got, ref, TAU[act])


# The matrix-core state passes run in one launch, each in a one-slice or a
# multi-slice form (the forward-state pass 4 or 2 value slices per
# workgroup, the reverse pass 2) chosen by the workgroup count of each form.
# These cases reach the multi-slice forms in the packed call and other forms
# in the per-sequence calls, and compare with the oracle and, bit for bit,
# across the two.
MULTI = [
    ("slices4-dk128-fp16-8seq", 4, {"lengths": (1, 63, 64, 65, 130, 2, 3, 100)}),
    ("slices4-dk64-bf16-8seq", 4, {"act": "bf16", "dk": 64, "lengths": (70, 1, 64, 129, 5, 66, 30, 64)}),
    ("slices4-dk64-fp16-8seq", 4, {"dk": 64, "lengths": (3, 130, 64, 1, 65, 200, 63, 2)}),
    # 16 sequences of 8 value heads: the packed call takes the multi-slice
    # forms of both passes, each per-sequence call (8 pairs) the one-slice ones
    ("multi-vs-one-slice-dk128-bf16-16seq", 4,
     {"act": "bf16", "Hqk": 4, "Hv": 8,
      "lengths": (65, 1, 130, 64, 0, 200, 3, 127, 64, 66, 10, 129, 2, 70, 191, 33)}),
]


@pytest.mark.parametrize("name,cfg,over", MULTI, ids=[m[0] for m in MULTI])
def test_chunk_rule_bwd_multi_slice_states(name, cfg, over):
    s, q, k, v, g, beta, cu = _inputs(cfg, over)
    (qd, kd, vd, gd, bd), cud = _dev(s, (q, k, v, g, beta), cu)
    N = len(cu) - 1
    do = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 460).cuda()
    h0 = synth.randn((N, s.Hv, s.dv, s.dk), "f32", 461).cuda() * 0.5
    dfin = synth.randn((N, s.Hv, s.dv, s.dk), "f32", 462).cuda() * 0.5
    scale = s.dk ** -0.5
    got = gdn.gdn_chunk_rule_bwd(qd, kd, vd, gd, bd, do, scale, True, 1e-6, cud, h0, dfin,
                                 want_d_initial_state=True)
    torch.cuda.synchronize()
    ref = OB.chunk_rule_bwd(q, k, v, g, beta, f64(do), scale, True, 1e-6, cu, f64(h0), f64(dfin))
    _check(got, ref, TAU[s.act])
    for i in range(N):
        a, b = int(cu[i]), int(cu[i + 1])
        if a == b:
            assert torch.equal(got[5][i], dfin[i]), ("d_initial_state of an empty sequence", i)
            continue
        one = gdn.gdn_chunk_rule_bwd(qd[:, a:b], kd[:, a:b], vd[:, a:b], gd[:, a:b], bd[:, a:b], do[:, a:b], scale,
                                     True, 1e-6, None, h0[i:i + 1], dfin[i:i + 1], want_d_initial_state=True)
        torch.cuda.synchronize()
        for n, x, y in zip(NAMES[:5], got[:5], one[:5]):
            assert torch.equal(x[:, a:b], y), (n, i)
        assert torch.equal(got[5][i], one[5][0]), ("d_initial_state", i)


def test_chunk_rule_bwd_back_to_back_on_a_stream():
    """Two calls in a row on a non-default stream with one workspace (the
    two-slice state passes, launched together): every kernel of a call is
    ordered on the caller's stream, so the second call's prep cannot
    overwrite records the first call's passes still read. Both results equal
    the same calls made one at a time on the default stream."""
    s = synth.spec(3).replace(T=640, Hqk=16, Hv=32)
    dt = synth.TORCH_DTYPE[s.act]
    ins = []
    for seed in (0, 1):
        q = synth.randn((1, s.T, s.Hqk, s.dk), s.act, 480 + 10 * seed).cuda()
        k = synth.randn((1, s.T, s.Hqk, s.dk), s.act, 481 + 10 * seed).cuda()
        v = synth.randn((1, s.T, s.Hv, s.dv), s.act, 482 + 10 * seed).cuda()
        g = -torch.rand(1, s.T, s.Hv, generator=torch.Generator().manual_seed(483 + seed)).cuda() * 0.3
        b = torch.rand(1, s.T, s.Hv, generator=torch.Generator().manual_seed(484 + seed)).cuda()
        do = synth.randn((1, s.T, s.Hv, s.dv), s.act, 485 + 10 * seed).cuda()
        ins.append((q, k, v, g, b, do))
    ws = torch.empty(gdn.gdn_chunk_rule_bwd_workspace_bytes(1, s.T, (s.Hqk, s.dk, s.Hv, s.dv)), dtype=torch.uint8,
                     device="cuda")
    scale = s.dk ** -0.5
    ref = []
    for x in ins:
        ref.append([t.clone() for t in gdn.gdn_chunk_rule_bwd(*x[:5], x[5], scale, True, 1e-6, workspace=ws)
                    if t is not None])
        torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        got = [[t for t in gdn.gdn_chunk_rule_bwd(*x[:5], x[5], scale, True, 1e-6, workspace=ws) if t is not None]
               for x in ins]
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    assert dt in (torch.bfloat16, torch.float16)
    for i in range(2):
        for j, (a, r) in enumerate(zip(got[i], ref[i])):
            assert torch.equal(a, r), (i, NAMES[j])
