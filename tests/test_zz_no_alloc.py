"""gdn_chunk_rule_fwd_noalloc (chunk records in the library's static device
scratch, no allocation in the call) against gdn_chunk_rule_fwd with a caller
workspace: the same kernels on the same inputs, so the outputs must be
identical. Two calls in a row on the same device, the second with a smaller
input, so the second runs on scratch that still holds the first call's
records; a third call takes the single-kernel path (FP32, no scratch)."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_qkv_amd import gdn, synth
from oracle import gdn as O
from . import _gdn_helpers as H

pytestmark = pytest.mark.gpu


def _inputs(act, T, Hqk, dk, Hv, dv, seed, lengths=None):
    B = 1
    q = synth.randn((B, T, Hqk, dk), act, seed).cuda()
    k = synth.randn((B, T, Hqk, dk), act, seed + 1).cuda()
    v = synth.randn((B, T, Hv, dv), act, seed + 2).cuda()
    g = torch.from_numpy(O.round_to(-synth.uniform((B, T, Hv), 0.0, 0.3, seed + 3), "f32")).float().cuda()
    beta = torch.from_numpy(O.round_to(synth.uniform((B, T, Hv), 0.05, 1.0, seed + 4), "f32")).float().cuda()
    cu = None
    N = B
    if lengths is not None:
        c = np.zeros(len(lengths) + 1, dtype=np.int32)
        c[1:] = np.cumsum(lengths)
        cu = torch.from_numpy(c).cuda()
        N = len(lengths)
    S0 = (synth.randn((N, Hv, dv, dk), "f32", seed + 5) * 0.5).cuda()
    return q, k, v, g, beta, cu, S0


CASES = [
    # (act, T, Hqk, dk, Hv, dv, lengths): the largest first
    ("bf16", 8000, 8, 128, 16, 128, None),
    ("f16", 700, 2, 64, 4, 64, (0, 130, 1, 64, 505)),
    ("f32", 300, 2, 64, 4, 64, None),
]


def test_noalloc_entry_point_matches_workspace_entry_point():
    for i, (act, T, Hqk, dk, Hv, dv, lengths) in enumerate(CASES):
        print(f"[noalloc] call {i}: {act} T={T} {Hqk}x{dk} -> {Hv}x{dv} lengths={lengths}", flush=True)
        q, k, v, g, beta, cu, S0 = _inputs(act, T, Hqk, dk, Hv, dv, 700 + 10 * i, lengths)
        need = gdn.gdn_chunk_rule_workspace_bytes(1, T, (Hqk, dk, Hv, dv), q.dtype,
                                                  0 if cu is None else cu.shape[0] - 1)
        assert need <= gdn.GDN_NOALLOC_SCRATCH_BYTES
        scale = dk ** -0.5
        ref_o, ref_f = gdn.gdn_chunk_rule_fwd(q, k, v, g, beta, scale, True, 1e-6, cu, S0,
                                              output_final_state=True, workspace="auto")
        o = torch.full_like(ref_o, float("nan"))
        fin = torch.full_like(ref_f, float("nan"))
        gdn.gdn_chunk_rule_fwd_noalloc(q, k, v, g, beta, scale, True, 1e-6, cu, S0, out_o=o, final_state=fin)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), f"call {i}: o"
        assert torch.equal(fin, ref_f), f"call {i}: final state"
        # and against the oracle, to the parity bar
        ro, rf = O.gated_delta_rule(H.f64(q), H.f64(k), H.f64(v), H.f64(g), H.f64(beta), scale=scale,
                                    cu_seqlens=None if cu is None else cu.cpu().numpy().astype(np.int64),
                                    initial_state=H.f64(S0), output_final_state=True)
        H.assert_close(H.f64(o), O.round_to(ro, act), H.TAU[act], f"call {i}: o vs oracle")
        H.assert_close(H.f64(fin), rf, H.TAU[act], f"call {i}: final state vs oracle")
