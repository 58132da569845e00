"""bench.py's output contract on a small workload: one JSON line with the
metric, the whole-job value, the roofline of the dominant kernel and the CPU
oracle baseline, plus the decode and backward legs."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_emits_one_json_line_with_roofline_and_cpu_baseline():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "2", "--steps", "2",
                        "--warmup", "1", "--decode-seqs", "8", "--no-whole-layer", "--cpu-budget", "1",
                        "--other-workloads", "0", "--other-reps", "3"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["value"] > 0
    assert out["config"]["workload"] == "gqa-bf16-T8192"
    roof = out["roofline"]
    assert roof["bound"] in ("hbm", "mfma") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < roof["frac"] <= 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert out["decode"]["seqs"] == 8 and out["decode"]["GB/s"] > 0
    assert set(out["backward"]) == {"gated_norm_bwd", "prologue_bwd", "chunk_rule_bwd", "layer_core_bwd_ms",
                                    "layer_core_bwd_saved_ms", "layer_core_fwd_bwd_saved_ms"}
    for key in ("layer_core_bwd_ms", "layer_core_bwd_saved_ms", "layer_core_fwd_bwd_saved_ms"):
        assert out["backward"][key] > 0, key
    q = out["ms_per_step_q"]
    assert 0 < q["p20"] <= q["median"] <= q["p80"]
    (other,) = out["other_workloads"]
    assert other["workload"] == "tiny-fp32" and other["tokens/s"] > 0
    for st in ("prologue", "chunk_rule", "gated_norm"):
        assert other[st]["hbm_frac"] > 0 and other[st]["ms"]["median"] > 0
    rb = out["backward"]["chunk_rule_bwd"]
    assert rb["ms"] > 0 and 0 < rb["frac"] <= 1 and 0 < rb["fp32_vector_frac"]
    assert rb["arith"] in ("bf16 mfma, split operands", "f16 mfma, split operands", "f32 vector")
