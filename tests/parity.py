"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same inputs, compare element by element."""
import sys

import numpy as np
import torch

import flashattention_forward_fwd_amd as fa
from oracle import ref

# Acceptance bars (max-abs error against the float64 oracle).
TOL = {
    "bf16": {"o": 2e-2, "lse": 1e-3},
    "fp32": {"o": 1e-5, "lse": 1e-5},
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, causal, scale, num_splits=None):
    """q, k, v: CPU tensors.  Returns (o, lse) as float64 numpy arrays.
    num_splits None: one-pass kernel; an int: the split-KV path."""
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.forward(dq, dk, dv, causal=causal, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def widen(t):
    return t.to(torch.float64).numpy()


def compare(name, dtype, o_gpu, lse_gpu, o_ref, lse_ref):
    assert np.all(np.isfinite(o_gpu)), "%s: non-finite output" % name
    assert np.all(np.isfinite(lse_gpu)), "%s: non-finite lse" % name
    eo = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    el = float(np.max(np.abs(lse_gpu - lse_ref))) if lse_ref.size else 0.0
    say("  %-44s max|dO|=%.3e  max|dLSE|=%.3e" % (name, eo, el))
    assert eo <= TOL[dtype]["o"], "%s: O error %.3e > %.1e" % (name, eo, TOL[dtype]["o"])
    assert el <= TOL[dtype]["lse"], "%s: LSE error %.3e > %.1e" % (name, el, TOL[dtype]["lse"])
    return eo, el


def check_case(name, q, k, v, causal, scale, dtype, rows=None, num_splits=None):
    """Full or row-sampled comparison of the HIP path with the oracle."""
    say("case %s: B,H,Lq,Lk,d=%s causal=%d splits=%s"
        % (name, tuple(q.shape[:3]) + (k.shape[2], q.shape[3]), causal, num_splits))
    o_gpu, lse_gpu = run_gpu(q, k, v, causal, scale, num_splits)
    o_ref, lse_ref = ref.attention_f64(widen(q), widen(k), widen(v), scale, causal, rows=rows)
    if rows is not None:
        B, H = q.shape[:2]
        rows = np.asarray(rows).reshape(B * H, -1) if np.ndim(rows) == 2 else np.broadcast_to(rows, (B * H, len(rows)))
        o_gpu = np.stack([o_gpu[bh // H, bh % H, rows[bh]] for bh in range(B * H)]).reshape(o_ref.shape)
        lse_gpu = np.stack([lse_gpu[bh // H, bh % H, rows[bh]] for bh in range(B * H)]).reshape(lse_ref.shape)
    return compare(name, dtype, o_gpu, lse_gpu, o_ref, lse_ref)
