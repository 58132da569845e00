"""The C ABI driven from C alone: tests/c_abi/layer_from_c.c is compiled
against include/gdn.h, libgdn.so and the HIP runtime (no Python binding, no
PyTorch in that process), runs gdn_layer_fwd and gdn_decode_fwd on inputs
written here, and its outputs are checked against the FP64 oracle."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from linear_attention_rnn_qkv_amd import synth
from oracle import gdn as O
from . import _gdn_helpers as H

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_attention_rnn_qkv_amd")


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().tobytes()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_layer_and_decode_from_c(tmp_path):
    exe = tmp_path / "layer_from_c"
    subprocess.run(["gcc", "-O2", "-std=c11", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "c_abi", "layer_from_c.c"), "-L", PKG, "-lgdn", "-L", "/opt/rocm/lib",
                    "-lamdhip64", f"-Wl,-rpath,{PKG}", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)], check=True)
    s = synth.spec(3).replace(B=2, T=130, Hqk=2, Hv=4)
    x = synth.make_inputs(s)
    scale = s.dk ** -0.5
    hdr = np.array([s.B, s.T, s.Hqk, s.dk, s.Hv, s.dv], dtype="<i8").tobytes() + np.float32(scale).tobytes()
    body = b"".join(_bits(x[k]) for k in ("x_q", "x_k", "x_v", "conv_w", "a", "b", "gate", "norm_w"))
    body += x["A_log"].numpy().astype("<f4").tobytes() + x["dt_bias"].numpy().astype("<f4").tobytes()
    (tmp_path / "in.bin").write_bytes(hdr + body)
    r = subprocess.run([str(exe), str(tmp_path / "in.bin"), str(tmp_path / "out.bin")], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = (tmp_path / "out.bin").read_bytes()
    n_out, n_dec = s.B * s.T * s.Hv * s.dv, s.B * s.Hv * s.dv
    bf = lambda b: torch.from_numpy(np.frombuffer(b, dtype=np.int16).copy()).view(torch.bfloat16)  # noqa: E731
    out = bf(raw[:2 * n_out]).reshape(s.B, s.T, s.Hv, s.dv)
    dec = bf(raw[2 * n_out:2 * (n_out + n_dec)]).reshape(s.B, s.Hv, s.dv)
    state = np.frombuffer(raw[2 * (n_out + n_dec):], dtype="<f4").reshape(s.B, s.Hv, s.dv, s.dk)
    tau = H.TAU[s.act]
    H.assert_close(H.f64(out), H.oracle_layer(x, s, scale), tau, "layer from C")
    f = synth.to_f64
    ro, _, rs = O.decode_step(f(x["x_q"])[:, 0], f(x["x_k"])[:, 0], f(x["x_v"])[:, 0], f(x["conv_w"]), None,
                              np.zeros((s.B, 3, s.C)), f(x["a"])[:, 0], f(x["b"])[:, 0], f(x["A_log"]),
                              f(x["dt_bias"]), np.zeros((s.B, s.Hv, s.dv, s.dk)), f(x["gate"])[:, 0],
                              f(x["norm_w"]), Hqk=s.Hqk, dk=s.dk, Hv=s.Hv, dv=s.dv, act=s.act, scale=scale)
    H.assert_close(H.f64(dec), ro, tau, "decode from C")
    H.assert_close(state.astype(np.float64), rs, tau, "decode state from C")
