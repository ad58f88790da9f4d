"""fa2_fwd_splitkv_static, the split-KV forward that allocates nothing (its
partial results live in the library's static device array), against
fa2_fwd_splitkv, the same path with a caller workspace.

Three calls of the static entry point in a row, each on a smaller input than
the one before, so a call that read partials left by the previous one would
show; each must give exactly the workspace path's result (same kernels, same
split count), hence also stay within the bf16 bars of the other parity tests.
"""
import ctypes

import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd.inputs import random_qkv
from tests.parity import TOL, say

# (B, H, Lq, Lk, d, causal, num_splits): MFMA partial kernel with 4 ranges; causal,
# automatic count; the decoding kernel (3 query rows), automatic count.
CASES = [
    (2, 4, 300, 5000, 128, False, 4),
    (1, 4, 700, 700, 128, True, 0),
    (1, 2, 3, 2000, 64, False, 0),
]


def _scale(d):
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


def _outputs(q):
    B, H, Lq, _ = q.shape
    return torch.full_like(q, float("nan")), torch.full((B, H, Lq), float("nan"), device=q.device)


@pytest.mark.gpu
def test_static_scratch_matches_workspace_path():
    stream = torch.cuda.current_stream().cuda_stream
    inputs, want = [], []
    for i, (B, H, Lq, Lk, d, causal, S) in enumerate(CASES):
        q, k, v = (t.cuda() for t in random_qkv(B, H, Lq, Lk, d, "bf16", seed=700 + i))
        o, lse = _outputs(q)
        ws = torch.empty(fa.fa2_splitkv_workspace_bytes(B, H, Lq, Lk, d, int(causal), S), dtype=torch.uint8,
                         device="cuda")
        fa.fa2_fwd_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, _scale(d), int(causal), S, ws, ws.numel(), stream)
        inputs.append((q, k, v))
        want.append((o, lse))
    torch.cuda.synchronize()
    outs = [_outputs(q) for q, _, _ in inputs]
    # warm-up: loads the library's code objects (and its static array) on this device
    q, k, v = inputs[-1]
    fa.fa2_fwd_splitkv_static(q, k, v, *_outputs(q), *CASES[-1][:5], _scale(CASES[-1][4]), 0, 0, stream)
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]
    for i, ((B, H, Lq, Lk, d, causal, S), (q, k, v), (o, lse)) in enumerate(zip(CASES, inputs, outs)):
        say("case static-scratch split-KV call %d: B,H,Lq,Lk,d=%s causal=%d num_splits=%d (resolved %d)"
            % (i, (B, H, Lq, Lk, d), causal, S, S or fa.fa2_splitkv_num_splits(B, H, Lq, Lk, d, int(causal))))
        fa.fa2_fwd_splitkv_static(q, k, v, o, lse, B, H, Lq, Lk, d, _scale(d), int(causal), S, stream)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free_before, "device memory changed across the calls"
    for i, ((o, lse), (wo, wl)) in enumerate(zip(outs, want)):
        eo = float((o.float() - wo.float()).abs().max())
        el = float((lse - wl).abs().max())
        say("  call %d: max|dO| vs workspace path %.3e, max|dLSE| %.3e" % (i, eo, el))
        assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]
        assert torch.equal(o, wo) and torch.equal(lse, wl), "static-scratch result differs from the workspace path"


def test_static_scratch_size_rejected_before_any_hip_call():
    """Partials larger than FA2_STATIC_SCRATCH_BYTES: FA2_ERR_SCRATCH, decided from the
    sizes alone when num_splits > 0 (stand-in aligned addresses are never touched)."""
    B, H, Lq, Lk, d, S = 4, 32, 4096, 4096, 128, 2
    assert fa.fa2_splitkv_workspace_bytes(B, H, Lq, Lk, d, 1, S) > fa.FA2_STATIC_SCRATCH_BYTES
    p = ctypes.c_void_p(1 << 20)
    st = fa.lib().fa2_fwd_splitkv_static(p, p, p, p, p, B, H, Lq, Lk, d, 0.088, 1, S, None)
    assert st == 9, fa.status_string(st)
    assert "static scratch" in fa.status_string(9)
    # num_splits out of range is FA2_ERR_ARG, as for fa2_fwd_splitkv
    assert fa.lib().fa2_fwd_splitkv_static(p, p, p, p, p, 1, 1, 64, 64, 64, 0.125, 0, -1, None) == 4
