"""Benchmark of the GDN layer-core forward on one MI355X.

One step = one pass of the whole layer core (prologue -> chunked gated delta
rule -> gated RMSNorm) over one batch of synthetic input resident in HBM.
Default workload: long-bf16-T131072 (B=1, 131072 tokens, 16 q/k heads of 128,
32 value heads of 128, chunk 64), the configuration the roofline fractions of
the stages are defined on. ``--config 0..4`` selects another workload.

Prints one JSON line: whole-job tokens/s, per-stage times and roofline
fractions measured with HIP events on the stream the kernels run on, the
dominant kernel's roofline, and the FP64 CPU oracle timed on a bounded sample
of the same workload on this machine's host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN layer-core fwd tokens/s at 1 GPU; % of HBM BW / MFMA peak per stage"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
FP32_VECTOR_PEAK_TFLOPS = 157.3
CHUNK = 64


def stage_work(s) -> dict:
    """Algorithmic bytes / flops per token of each stage (no recompute)."""
    e = {"f32": 4, "bf16": 2, "f16": 2}[s.act]
    eg = {"f32": 4, "bf16": 2, "f16": 2}[s.gate_dtype]
    C = s.C
    return {
        # read x (C channels) and a, b; write qkv (C) and g, beta (FP32)
        "prologue_bytes": 2 * C * e + 2 * s.Hv * e + 8 * s.Hv,
        # read q, k, v, g, beta; write o
        "chunk_bytes": (2 * s.Hqk * s.dk + 2 * s.Hv * s.dv) * e + 8 * s.Hv,
        "chunk_flops": s.Hv * (6 * CHUNK * s.dk + 4 * CHUNK * s.dv + 6 * s.dk * s.dv),
        # read o and gate, write out
        "norm_bytes": s.Hv * s.dv * (2 * e + eg),
    }


def cpu_baseline(cfg: int, s, budget_s: float) -> dict:
    """The FP64 oracle (as it stands) on a prefix of the workload's tokens."""
    import numpy as np

    from linear_attention_rnn_qkv_amd import synth
    from oracle import gdn as O

    threads = O.default_threads()
    # calibrate on a short prefix, then run a prefix sized to the budget
    def run(ntok):
        sub = s.replace(T=ntok, B=1, lengths=None)
        x = synth.make_inputs(sub)
        f = synth.to_f64
        t0 = time.perf_counter()
        O.layer(f(x["x_q"]), f(x["x_k"]), f(x["x_v"]), f(x["conv_w"]), None, f(x["a"]), f(x["b"]),
                f(x["A_log"]), f(x["dt_bias"]), f(x["gate"]), f(x["norm_w"]), Hqk=s.Hqk, dk=s.dk,
                Hv=s.Hv, dv=s.dv, act=s.act, scale=s.dk ** -0.5, threads=threads)
        return time.perf_counter() - t0

    t_cal = run(256)
    ntok = int(min(s.T, max(256, 256 * budget_s / max(t_cal, 1e-3))))
    ntok = max(256, ntok // 64 * 64)
    dt = run(ntok)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {ntok} tokens of one sequence of workload {s.name}, all {s.Hv} value "
                      f"heads, whole layer core (FP64 C recurrence + NumPy stages), {dt:.1f} s",
            "cpu": cpu}


COPY_BYTES = 1 << 30


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch (summed over the '+'-joined kernels of a stage) from
    the committed rocprofv3 counter summary of this workload, if it was taken
    on the kernels' current sources; else None."""
    from linear_attention_rnn_qkv_amd import profile_summary as ps

    path = os.path.join(ROOT, "profiles", f"hbm_traffic.{workload}.json")
    try:
        with open(path) as fh:
            recs = json.load(fh)["kernels"]
    except (OSError, KeyError, ValueError):
        return None
    total = 0.0
    for k in kernel.split("+"):
        rec = recs.get(k)
        if rec is None or k not in ps.KERNELS or rec.get("source_hash") != ps.source_hash(k):
            return None
        total += rec["bytes"]
    return total


def quantiles(ts) -> dict:
    """Median and 20th / 80th percentiles (ms) of per-call times."""
    ts = sorted(ts)
    q = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]  # noqa: E731
    return {"median": q(0.5), "p20": q(0.2), "p80": q(0.8)}


def mfma_counters(workload: str, kernel: str):
    """Counter-based MFMA utilisation of a ('+'-joined) stage from the
    committed rocprofv3 summary of this workload, if it was taken on the
    kernels' current sources; else None. Per kernel: SQ_VALU_MFMA_BUSY_CYCLES
    / (GRBM_GUI_ACTIVE x CUs), the fraction of the launch during which the
    matrix cores were busy; the stage value weights the kernels by their
    average durations."""
    from linear_attention_rnn_qkv_amd import profile_summary as ps

    path = os.path.join(ROOT, "profiles", f"mfma_counters.{workload}.json")
    try:
        with open(path) as fh:
            recs = json.load(fh)["kernels"]
    except (OSError, KeyError, ValueError):
        return None
    num = den = 0.0
    for k in kernel.split("+"):
        rec = recs.get(k)
        if rec is None or k not in ps.KERNELS or rec.get("source_hash") != ps.source_hash(k):
            return None
        num += rec["mfma_busy"] * rec["avg_us"]
        den += rec["avg_us"]
    return num / den if den else None


def stage_times(gdn, synth, torch, cfg: int, reps: int, flush_bytes: int = 512 << 20) -> dict:
    """Per-stage and whole-layer times of workload ``cfg`` (median and
    quantiles over ``reps`` calls, a 512 MB write before each call so that
    no stage reads its inputs from the 256 MB Infinity Cache), with bytes and
    roofline fractions. Used for the workloads beside the headline one."""
    s = synth.spec(cfg)
    print(f"[bench] stage times, workload {cfg} {s.name}", file=sys.stderr, flush=True)
    x = synth.make_inputs(s)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    del x
    dims = (s.Hqk, s.dk, s.Hv, s.dv)
    scale = s.dk ** -0.5
    dt = synth.TORCH_DTYPE[s.act]
    n_seqs = 0 if d["cu_seqlens"] is None else d["cu_seqlens"].shape[0] - 1
    ws = torch.empty(gdn.gdn_layer_workspace_bytes(s.B, s.T, dims, dt, n_seqs), dtype=torch.uint8, device="cuda")
    cws_bytes = gdn.gdn_chunk_rule_workspace_bytes(s.B, s.T, dims, dt, n_seqs)
    cws = torch.empty(cws_bytes, dtype=torch.uint8, device="cuda") if cws_bytes else None
    out = torch.empty((s.B, s.T, s.Hv, s.dv), dtype=dt, device="cuda")
    qkv = torch.empty((s.B, s.T, s.C), dtype=dt, device="cuda")
    g = torch.empty((s.B, s.T, s.Hv), dtype=torch.float32, device="cuda")
    beta = torch.empty_like(g)
    o = torch.empty((s.B, s.T, s.Hv, s.dv), dtype=dt, device="cuda")
    nq = s.Hqk * s.dk
    qv = qkv[..., :nq].unflatten(-1, (s.Hqk, s.dk))
    kv = qkv[..., nq:2 * nq].unflatten(-1, (s.Hqk, s.dk))
    vv = qkv[..., 2 * nq:].unflatten(-1, (s.Hv, s.dv))
    calls = {
        "layer": lambda: gdn.gdn_layer_fwd(d["x_q"], d["x_k"], d["x_v"], d["conv_w"], None, d["a"], d["b"],
                                           d["A_log"], d["dt_bias"], d["gate"], d["norm_w"], d["cu_seqlens"],
                                           dims, scale, workspace=ws, out=out),
        "prologue": lambda: gdn.gdn_prologue_fwd(d["x_q"], d["x_k"], d["x_v"], d["conv_w"], None, d["a"], d["b"],
                                                 d["A_log"], d["dt_bias"], d["cu_seqlens"], dims, out_qkv=qkv,
                                                 out_g=g, out_beta=beta),
        "chunk_rule": lambda: gdn.gdn_chunk_rule_fwd(qv, kv, vv, g, beta, scale, True, 1e-6, d["cu_seqlens"],
                                                     out_o=o, workspace=cws),
        "gated_norm": lambda: gdn.gdn_gated_norm_fwd(o, d["gate"], d["norm_w"], 1e-5, out=out),
    }
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    res = {}
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[name] = quantiles(ts)
    w = stage_work(s)
    n = s.tokens
    out_d = {"workload": s.name, "tokens": n, "reps": reps,
             "layer_ms": res["layer"], "tokens/s": n / (res["layer"]["median"] * 1e-3)}
    for name, key in (("prologue", "prologue_bytes"), ("chunk_rule", "chunk_bytes"), ("gated_norm", "norm_bytes")):
        t = res[name]["median"]
        gb = w[key] * n / (t * 1e-3) / 1e9
        out_d[name] = {"ms": res[name], "GB/s": gb, "hbm_frac": gb / HBM_PEAK_GBS}
        if name == "chunk_rule":
            out_d[name]["TFLOP/s"] = w["chunk_flops"] * n / (t * 1e-3) / 1e12
            out_d[name]["mfma_frac"] = out_d[name]["TFLOP/s"] / MFMA_PEAK_TFLOPS[s.act]
    del ws, cws, qkv, o, out, d
    torch.cuda.empty_cache()
    return out_d


def calibrate_copy(reps: int) -> int:
    """A plain device copy of COPY_BYTES, `reps` times: its byte counters per
    dispatch (which must read COPY_BYTES fetched and written) calibrate the
    HBM traffic counters of the kernels."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"calibration": "device copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                      "ms": ms, "GB/s": 2 * COPY_BYTES / (ms * 1e-3) / 1e9}), flush=True)
    return 0


def decode_leg(gdn, synth, torch, s, d, dims, scale, N, steps, warmup) -> dict:
    """The recurrent decode step (one token for each of N sequences, conv
    cache and FP32 state updated in place) at the workload's head geometry.
    Not the headline metric: reported beside it, against the HBM roof (the
    state is read and written once per step)."""
    dt = synth.TORCH_DTYPE[s.act]
    e = {"f32": 4, "bf16": 2, "f16": 2}[s.act]
    eg = {"f32": 4, "bf16": 2, "f16": 2}[s.gate_dtype]
    tok = synth.make_inputs(s.replace(B=N, T=1, lengths=None, gate_in_proj=False))
    t = {k: tok[k][:, 0].contiguous().cuda() for k in ("x_q", "x_k", "x_v", "a", "b", "gate")}
    cache = synth.randn((N, 3, s.C), s.act, 7).cuda()
    state = (0.5 * synth.randn((N, s.Hv, s.dv, s.dk), "f32", 8)).cuda()
    out = torch.empty((N, s.Hv, s.dv), dtype=dt, device="cuda")

    def step():
        gdn.gdn_decode_fwd(t["x_q"], t["x_k"], t["x_v"], d["conv_w"], None, cache, t["a"], t["b"],
                           d["A_log"], d["dt_bias"], state, t["gate"], d["norm_w"], dims, scale, out=out)

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # per sequence: state read + written (FP32), x, conv cache read + written,
    # a and b, gate, out; per launch: conv weights and norm weight
    per_seq = (2 * s.Hv * s.dv * s.dk * 4 + s.C * e + 6 * s.C * e + 2 * s.Hv * e + s.Hv * s.dv * (eg + e))
    nbytes = N * per_seq + 4 * s.C * e + s.dv * e
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "decode_kernel", "seqs": N, "ms": ms, "bytes": nbytes, "GB/s": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS, "tokens/s": N / (ms * 1e-3)}


# The pages' whole-layer shapes (flash-linear-attention GatedDeltaNet with
# num_heads=6, expand_v=2; page "fused q/k/v short conv", Benchmark /
# Performance) and their B200 forward times with the fused conv, as context.
WHOLE_LAYER_SHAPES = [  # (B, T, hidden, head_dim, act, B200 fused fwd ms, B200 fused fwd+bwd ms)
    (2, 2048, 2048, 256, "bf16", 1.540, 4.084),
    (1, 128, 512, 64, "bf16", 1.493, 4.066),
    (2, 100, 512, 64, "bf16", 1.486, 4.088),
    (2, 256, 512, 64, "f16", 1.488, 4.095),
]


def chunk_bwd_flops(s) -> float:
    """Algorithmic FLOPs of the chunk-rule backward: per (chunk of C = 64
    tokens, value head), 2 (8 C dk dv + 5 C^2 dv + 4 C^2 dk + 2 C^2 dk / G
    + C^3 / 3): the state checkpoints (K S0^T, M X, the state update), the
    reverse pass (P^T dO, K dS^T, M^T dDelta, two state-gradient products),
    the per-chunk gradients (two C x C and three C x dk contractions over dv,
    four C x dk contractions over the chunk, q.k and k.k per q/k head) and
    the triangular inverse. Ragged chunks count as full ones."""
    C, G = 64, s.Hv // s.Hqk
    lens = s.lengths if s.lengths is not None else (s.T,) * s.B
    chunks = sum((L + C - 1) // C for L in lens)
    per = 2 * (8 * C * s.dk * s.dv + 5 * C * C * s.dv + 4 * C * C * s.dk + 2 * C * C * s.dk / G + C ** 3 / 3)
    return chunks * s.Hv * per


def backward_leg(gdn, synth, torch, s, d, o, dims, steps, warmup, rule=None, layer=True) -> dict:
    """The backward calls at the workload's shape: per-call HIP events on the
    current stream, mean over `steps` calls. The gated norm and the prologue
    are priced against the HBM roof (algorithmic bytes per token: norm
    Hv dv (3 e + 2 e_g) (o, dout, d_o; gate, d_gate); prologue
    3 C e + 4 Hv e + 8 Hv (x, d_qkv, dx; a, b, d_a, d_b; d_g, d_beta)); the
    chunk-rule backward with chunk_bwd_flops against the peak of the
    arithmetic it runs on (the 16-bit matrix cores with split operands for
    BF16 and FP16 at dk 64/128, else the FP32 vector peak), and against the FP32 vector
    peak for comparison. `rule` = (q, k, v, g, beta, scale) views of
    the forward's prologue output."""
    e = {"f32": 4, "bf16": 2, "f16": 2}[s.act]
    eg = {"f32": 4, "bf16": 2, "f16": 2}[s.gate_dtype]
    ntok = s.tokens
    dims_t = (s.Hqk, s.dk, s.Hv, s.dv)
    dout = synth.randn((s.B, s.T, s.Hv, s.dv), s.act, 61).cuda()
    dqkv = synth.randn((s.B, s.T, s.C), s.act, 62).cuda()
    dg = synth.randn((s.B, s.T, s.Hv), "f32", 63).cuda()
    dbeta = synth.randn((s.B, s.T, s.Hv), "f32", 64).cuda()
    nws = torch.empty(gdn.lib().gdn_gated_norm_bwd_workspace_bytes(s.B, s.T, s.Hv, s.dv), dtype=torch.uint8,
                      device="cuda")
    pws = torch.empty(gdn.lib().gdn_prologue_bwd_workspace_bytes(s.B, s.T, gdn.dims_of(*dims_t)),
                      dtype=torch.uint8, device="cuda")

    def norm_b():
        gdn.gdn_gated_norm_bwd(o, d["gate"], d["norm_w"], dout, 1e-5, workspace=nws)

    def pro_b():
        gdn.gdn_prologue_bwd(d["x_q"], d["x_k"], d["x_v"], d["conv_w"], None, d["a"], d["b"], d["A_log"],
                             d["dt_bias"], d["cu_seqlens"], dims, dqkv, dg, dbeta, workspace=pws)

    legs = [("gated_norm_bwd", norm_b, s.Hv * s.dv * (3 * e + 2 * eg)),
            ("prologue_bwd", pro_b, 3 * s.C * e + 4 * s.Hv * e + 8 * s.Hv)]
    out = {}
    if rule is not None and s.dk in (64, 128, 256):
        q, k, v, g, beta, scale = rule
        n_seqs = 0 if d["cu_seqlens"] is None else d["cu_seqlens"].shape[0] - 1
        rws = torch.empty(gdn.gdn_chunk_rule_bwd_workspace_bytes(s.B, s.T, dims_t, n_seqs), dtype=torch.uint8,
                          device="cuda")

        def rule_b():
            gdn.gdn_chunk_rule_bwd(q, k, v, g, beta, dout, scale, True, 1e-6, d["cu_seqlens"], workspace=rws)

        legs.append(("chunk_rule_bwd", rule_b, None))
    stream = torch.cuda.current_stream()
    for name, fn, per_tok in legs:
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        if per_tok is None:
            fl = chunk_bwd_flops(s)
            tf = fl / (ms * 1e-3) / 1e12
            # BF16 and FP16 workloads at dk 64/128 run the matrix-core kernels
            # (FP32 operands split into 16-bit hi + lo parts, about three MFMA
            # products per FP32 product); the rest run FP32 vector arithmetic
            mma = s.act in ("bf16", "f16") and s.dk in (64, 128)
            peak = MFMA_PEAK_TFLOPS[s.act] if mma else FP32_VECTOR_PEAK_TFLOPS
            out[name] = {"ms": ms, "flops": fl, "TFLOP/s": tf,
                         "arith": f"{s.act} mfma, split operands" if mma else "f32 vector",
                         "peak_TFLOP/s": peak,
                         "frac": tf / peak,
                         "fp32_vector_frac": tf / FP32_VECTOR_PEAK_TFLOPS}
            continue
        nbytes = per_tok * ntok
        out[name] = {"ms": ms, "bytes": nbytes, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                     "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if layer and s.dk in (64, 128, 256):
        # the whole layer-core backward in one call (its forward stages recomputed)
        scale = rule[5] if rule is not None else s.dk ** -0.5
        n_seqs = 0 if d["cu_seqlens"] is None else d["cu_seqlens"].shape[0] - 1
        lws = torch.empty(gdn.gdn_layer_bwd_workspace_bytes(s.B, s.T, dims_t, dout.dtype, n_seqs),
                          dtype=torch.uint8, device="cuda")

        def layer_b():
            gdn.gdn_layer_bwd(d["x_q"], d["x_k"], d["x_v"], d["conv_w"], None, d["a"], d["b"], d["A_log"],
                              d["dt_bias"], d["gate"], d["norm_w"], d["cu_seqlens"], dims, scale, dout, workspace=lws)

        for _ in range(warmup):
            layer_b()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            layer_b()
        e1.record(stream)
        torch.cuda.synchronize()
        out["layer_core_bwd_ms"] = e0.elapsed_time(e1) / steps

        # a training step of the core that keeps the forward's activations:
        # gdn_layer_fwd into the backward's workspace, then gdn_layer_bwd_saved
        # (no forward recompute); and that backward alone
        lo = torch.empty((s.B, s.T, s.Hv, s.dv), dtype=dout.dtype, device="cuda")
        fargs = (d["x_q"], d["x_k"], d["x_v"], d["conv_w"], None, d["a"], d["b"], d["A_log"], d["dt_bias"],
                 d["gate"], d["norm_w"], d["cu_seqlens"], dims, scale)

        def layer_f():
            gdn.gdn_layer_fwd(*fargs, workspace=lws, out=lo)

        def layer_bs():
            gdn.gdn_layer_bwd_saved(*fargs, dout, lws)

        for name, fns in (("layer_core_fwd_bwd_saved_ms", (layer_f, layer_bs)), ("layer_core_bwd_saved_ms",
                                                                                 (layer_bs,))):
            layer_f()
            for _ in range(warmup):
                for fn in fns:
                    fn()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(steps):
                for fn in fns:
                    fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out[name] = e0.elapsed_time(e1) / steps
        del lws, lo
    return out


def whole_layer_leg(gdn, synth, torch) -> list:
    """The whole layer forward: one input-projection GEMM to the fused
    q|k|v|gate|b|a buffer, the layer core on views of it, the output-projection
    GEMM; and forward + backward (fwdbwd_ms): the backward of a summed output
    through the output GEMM, gdn_layer_bwd, and the input GEMM's input and
    weight gradients. The GEMMs are plain library GEMMs (torch.matmul, which runs
    hipBLASLt/rocBLAS); the core is this library. Timed like the pages'
    script: untimed calls, then per-call HIP events with the caches flushed by
    a 512 MB write before each call, median of 200 calls."""
    res = []
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for i, (B, T, Hd, hd, act, b200, b200_fb) in enumerate(WHOLE_LAYER_SHAPES):
        Hqk, dk, Hv, dv = 6, hd, 6, 2 * hd
        nq, nv = Hqk * dk, Hv * dv
        C = 2 * nq + nv
        width = 2 * nq + 2 * nv + 2 * Hv
        dt = synth.TORCH_DTYPE[act]
        seed = 900 + 10 * i
        x = synth.randn((B, T, Hd), act, seed).cuda()
        w_in = (synth.randn((Hd, width), "f32", seed + 1) * Hd ** -0.5).to(dt).cuda()
        w_out = (synth.randn((nv, Hd), "f32", seed + 2) * nv ** -0.5).to(dt).cuda()
        conv_w = torch.from_numpy(synth.uniform((C, 4), -0.5, 0.5, seed + 3)).to(dt).cuda()
        A_log = torch.from_numpy(synth.uniform((Hv,), 1.0, 16.0, seed + 4)).log().float().cuda()
        dt_bias = (0.1 * synth.randn((Hv,), "f32", seed + 5)).cuda()
        norm_w = torch.ones(dv, dtype=dt, device="cuda")
        dims = (Hqk, dk, Hv, dv)
        ws = torch.empty(gdn.gdn_layer_workspace_bytes(B, T, dims, dt), dtype=torch.uint8, device="cuda")
        core = torch.empty((B, T, Hv, dv), dtype=dt, device="cuda")

        def fwd():
            proj = torch.matmul(x, w_in)
            o = 0
            xq = proj[..., o:o + nq]; o += nq
            xk = proj[..., o:o + nq]; o += nq
            xv = proj[..., o:o + nv]; o += nv
            gate = proj[..., o:o + nv].unflatten(-1, (Hv, dv)); o += nv
            b = proj[..., o:o + Hv]; o += Hv
            a = proj[..., o:o + Hv]
            gdn.gdn_layer_fwd(xq, xk, xv, conv_w, None, a, b, A_log, dt_bias, gate, norm_w, None, dims,
                              dk ** -0.5, workspace=ws, out=core)
            return torch.matmul(core.flatten(-2), w_out)

        def core_call():
            proj = proj_buf
            o = 0
            xq = proj[..., o:o + nq]; o += nq
            xk = proj[..., o:o + nq]; o += nq
            xv = proj[..., o:o + nv]; o += nv
            gate = proj[..., o:o + nv].unflatten(-1, (Hv, dv)); o += nv
            b = proj[..., o:o + Hv]; o += Hv
            a = proj[..., o:o + Hv]
            gdn.gdn_layer_fwd(xq, xk, xv, conv_w, None, a, b, A_log, dt_bias, gate, norm_w, None, dims,
                              dk ** -0.5, workspace=ws, out=core_out)

        def median_ms(fn):
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(200):
                flush.zero_()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ts.sort()
            return ts[len(ts) // 2]

        # forward and backward of the layer, as the pages' fwd+bwd timing runs
        # layer(x).sum().backward(): d(sum) = 1 at the output; the backward
        # recomputes the core's forward (gdn_layer_bwd), then the projection
        # GEMMs' input and weight gradients
        lws = torch.empty(gdn.gdn_layer_bwd_workspace_bytes(B, T, dims, dt), dtype=torch.uint8, device="cuda")
        w_in_t, w_out_t = w_in.t().contiguous(), w_out.t().contiguous()
        x_t = x.flatten(0, 1).t().contiguous()
        d_y = torch.ones((B, T, Hd), dtype=dt, device="cuda")

        def fwdbwd():
            proj = torch.matmul(x, w_in)
            o = 0
            xq = proj[..., o:o + nq]; o += nq
            xk = proj[..., o:o + nq]; o += nq
            xv = proj[..., o:o + nv]; o += nv
            gate = proj[..., o:o + nv].unflatten(-1, (Hv, dv)); o += nv
            b = proj[..., o:o + Hv]; o += Hv
            a = proj[..., o:o + Hv]
            gdn.gdn_layer_fwd(xq, xk, xv, conv_w, None, a, b, A_log, dt_bias, gate, norm_w, None, dims,
                              dk ** -0.5, workspace=ws, out=core)
            torch.matmul(core.flatten(-2), w_out)
            d_core = torch.matmul(d_y, w_out_t).unflatten(-1, (Hv, dv))
            torch.matmul(core.flatten(0, 1).flatten(-2).t().contiguous(), d_y.flatten(0, 1))  # d w_out
            g = gdn.gdn_layer_bwd(xq, xk, xv, conv_w, None, a, b, A_log, dt_bias, gate, norm_w, None, dims,
                                  dk ** -0.5, d_core, workspace=lws)
            d_proj = torch.cat([g[0], g[1], g[2], g[9].flatten(-2), g[6], g[5]], -1)
            torch.matmul(d_proj, w_in_t)  # d x
            torch.matmul(x_t, d_proj.flatten(0, 1))  # d w_in

        ms = median_ms(fwd)
        fb_ms = median_ms(fwdbwd)
        # the layer core alone on the same projection buffer
        proj_buf = torch.matmul(x, w_in)
        core_out = torch.empty((B, T, Hv, dv), dtype=dt, device="cuda")
        core_ms = median_ms(core_call)
        res.append({"shape": f"B{B}-T{T}-H{Hd}-hd{hd}", "dtype": act, "ms": ms, "tokens/s": B * T / (ms * 1e-3),
                    "pages_b200_fwd_ms": b200, "core_ms": core_ms, "fwdbwd_ms": fb_ms,
                    "pages_b200_fwdbwd_ms": b200_fb})
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-seqs", type=int, default=256,
                    help="sequences of the decode-step leg (0 skips it)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-whole-layer", action="store_true",
                    help="skip the whole-layer leg (projection GEMMs + layer core)")
    ap.add_argument("--no-layer-bwd", action="store_true",
                    help="skip the one-call layer-core backward (its prologue backward reads an FP32 d_qkv, "
                         "so per-kernel counter averages would mix two workloads)")
    ap.add_argument("--other-workloads", default="2,4",
                    help="comma-separated workloads whose per-stage fractions are reported beside the headline "
                         "one (median of --other-reps calls with the caches flushed before each); '' skips")
    ap.add_argument("--other-reps", type=int, default=30)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (got --gpus {args.gpus}); the layer core "
              "shards by heads or sequences without a collective, which is not built here.",
              file=sys.stderr)
        return 2

    import torch

    from linear_attention_rnn_qkv_amd import gdn, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        return calibrate_copy(args.steps)
    s = synth.spec(args.config)
    print(f"[bench] workload {args.config} {s.name}: generating inputs", file=sys.stderr, flush=True)
    x = synth.make_inputs(s)
    d = {}
    for k, v in x.items():
        d[k] = v.cuda() if isinstance(v, torch.Tensor) else v
    if x.get("proj") is not None:
        proj = x["proj"].cuda()
        for k in ("x_q", "x_k", "x_v", "gate", "b", "a"):
            v = x[k]
            d[k] = proj.as_strided(v.shape, v.stride(), v.storage_offset() - x["proj"].storage_offset())
    del x
    dims = (s.Hqk, s.dk, s.Hv, s.dv)
    scale = s.dk ** -0.5
    dt = synth.TORCH_DTYPE[s.act]
    n_seqs = 0 if d["cu_seqlens"] is None else d["cu_seqlens"].shape[0] - 1
    ws = torch.empty(gdn.gdn_layer_workspace_bytes(s.B, s.T, dims, dt, n_seqs), dtype=torch.uint8, device="cuda")
    cws_bytes = gdn.gdn_chunk_rule_workspace_bytes(s.B, s.T, dims, dt, n_seqs)
    cws = torch.empty(cws_bytes, dtype=torch.uint8, device="cuda") if cws_bytes else None
    out = torch.empty((s.B, s.T, s.Hv, s.dv), dtype=dt, device="cuda")
    # stage buffers for the per-stage timing loop (same kernels, same shapes)
    qkv = torch.empty((s.B, s.T, s.C), dtype=dt, device="cuda")
    g = torch.empty((s.B, s.T, s.Hv), dtype=torch.float32, device="cuda")
    beta = torch.empty_like(g)
    o = torch.empty((s.B, s.T, s.Hv, s.dv), dtype=dt, device="cuda")
    nq = s.Hqk * s.dk
    qv = qkv[..., :nq].unflatten(-1, (s.Hqk, s.dk))
    kv = qkv[..., nq:2 * nq].unflatten(-1, (s.Hqk, s.dk))
    vv = qkv[..., 2 * nq:].unflatten(-1, (s.Hv, s.dv))

    def layer():
        gdn.gdn_layer_fwd(d["x_q"], d["x_k"], d["x_v"], d["conv_w"], None, d["a"], d["b"], d["A_log"],
                          d["dt_bias"], d["gate"], d["norm_w"], d["cu_seqlens"], dims, scale, workspace=ws,
                          out=out)

    def prologue():
        gdn.gdn_prologue_fwd(d["x_q"], d["x_k"], d["x_v"], d["conv_w"], None, d["a"], d["b"], d["A_log"],
                             d["dt_bias"], d["cu_seqlens"], dims, out_qkv=qkv, out_g=g, out_beta=beta)

    def chunk():
        gdn.gdn_chunk_rule_fwd(qv, kv, vv, g, beta, scale, True, 1e-6, d["cu_seqlens"], out_o=o, workspace=cws)

    def norm():
        gdn.gdn_gated_norm_fwd(o, d["gate"], d["norm_w"], 1e-5, out=out)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer()
    torch.cuda.synchronize()

    # Timed region: exactly K steps of the layer core.
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step_ev[i].record(stream)
        layer()
    step_ev[args.steps].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    step_q = quantiles([step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps)])
    print(f"[bench] {args.steps} steps: {ms:.4f} ms/step", file=sys.stderr, flush=True)

    # Per-stage durations: the same three kernels, one event between each.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        e = evs[i]
        e[0].record(stream)
        prologue()
        e[1].record(stream)
        chunk()
        e[2].record(stream)
        norm()
        e[3].record(stream)
    torch.cuda.synchronize()
    q_pro = quantiles([e[0].elapsed_time(e[1]) for e in evs])
    q_chk = quantiles([e[1].elapsed_time(e[2]) for e in evs])
    q_nrm = quantiles([e[2].elapsed_time(e[3]) for e in evs])
    # stage time = the average launch duration (as the profiler reports it);
    # median and quantiles beside it
    t_pro = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    t_chk = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    t_nrm = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps

    w = stage_work(s)
    ntok = s.tokens
    pb, cb, cf, nb = (w["prologue_bytes"] * ntok, w["chunk_bytes"] * ntok, w["chunk_flops"] * ntok,
                      w["norm_bytes"] * ntok)
    mfma_peak = MFMA_PEAK_TFLOPS[s.act]

    def gbs(b, t_ms):
        return b / (t_ms * 1e-3) / 1e9

    # the chunk stage: chunk prep + chunk state (two launches) where a workspace
    # applies, else the single recurrence kernel
    chunk_kernel = ("chunk_rule_kernel" if cws is None else
                    "chunk_prep_kernel+chunk_state_wide_kernel" if s.dk == 256 else
                    "chunk_prep_kernel+chunk_state_kernel")
    stages = {
        "prologue": {"kernel": "prologue_kernel", "ms": t_pro, "ms_q": q_pro, "bytes": pb, "GB/s": gbs(pb, t_pro),
                     "hbm_frac": gbs(pb, t_pro) / HBM_PEAK_GBS},
        "chunk_rule": {"kernel": chunk_kernel, "ms": t_chk, "ms_q": q_chk, "bytes": cb, "flops": cf,
                       "GB/s": gbs(cb, t_chk), "hbm_frac": gbs(cb, t_chk) / HBM_PEAK_GBS,
                       "TFLOP/s": cf / (t_chk * 1e-3) / 1e12,
                       "mfma_frac": cf / (t_chk * 1e-3) / 1e12 / mfma_peak},
        "gated_norm": {"kernel": "gated_norm_kernel", "ms": t_nrm, "ms_q": q_nrm, "bytes": nb,
                       "GB/s": gbs(nb, t_nrm),
                       "hbm_frac": gbs(nb, t_nrm) / HBM_PEAK_GBS},
    }
    # dominant kernel and the roof that bounds it in the ideal
    dom = max(stages, key=lambda k: stages[k]["ms"])
    st = stages[dom]
    if dom == "chunk_rule" and cf / (mfma_peak * 1e12) > cb / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": st["TFLOP/s"], "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": st["mfma_frac"]}
    else:
        roof = {"bound": "hbm", "achieved": st["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": st["hbm_frac"]}
    roof["kernel"] = st["kernel"]
    roof["traffic"] = measured_traffic(s.name, st["kernel"])
    if dom == "chunk_rule":
        # matrix-core busy fraction from rocprofv3 counters (None if the
        # committed counters were taken on other sources)
        roof["mfma_util"] = mfma_counters(s.name, st["kernel"])
    for v in stages.values():
        v["traffic"] = measured_traffic(s.name, v["kernel"])

    decode = None
    if args.decode_seqs > 0:
        decode = decode_leg(gdn, synth, torch, s, d, dims, scale, args.decode_seqs, args.steps,
                            args.warmup)

    backward = None
    if not args.no_backward:
        print("[bench] backward leg", file=sys.stderr, flush=True)
        backward = backward_leg(gdn, synth, torch, s, d, o, dims, args.steps, args.warmup,
                                rule=(qv, kv, vv, g, beta, scale), layer=not args.no_layer_bwd)

    others = None
    if args.other_workloads:
        others = [stage_times(gdn, synth, torch, int(c), args.other_reps) for c in args.other_workloads.split(",")
                  if c.strip() and int(c) != args.config]

    whole = None
    if not args.no_whole_layer:
        print("[bench] whole-layer leg", file=sys.stderr, flush=True)
        whole = whole_layer_leg(gdn, synth, torch)

    result = {
        "metric": METRIC,
        "value": ntok / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_q": step_q,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.act,
        "data": "synthetic",
        "config": {"workload": s.name, "B": s.B, "T": s.T, "tokens": ntok, "Hqk": s.Hqk, "dk": s.dk,
                   "Hv": s.Hv, "dv": s.dv, "chunk": CHUNK, "conv_taps": 4, "parallelism": "single GPU"},
        "roofline": roof,
        "stages": stages,
        "other_workloads": others,
        "decode": decode,
        "whole_layer": whole,
        "backward": backward,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.config, s, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
