"""Parity of the fp16 entry points (fa2_fwd_f16, fa2_bwd_f16, through the C ABI)
with the float64 oracles.

Bars: fp16 rounds to 11 significant bits (bf16: 8), so the bf16 bars are halved:
max|O - O_ref| <= 1e-2, max|LSE - LSE_ref| <= 1e-3, and for each gradient G
max|G - G_ref| <= 1e-2 * max(1, max|G_ref|).  Worst-case derivation for O: half
an fp16 ulp of the output (2^-11 |O|, |O| <= max|V| ~ 4.5: 2.2e-3) plus the
rounding of the probabilities before P V (2^-11 relative, the same bound) --
about 4.4e-3, so 1e-2 leaves a factor of two.
"""
import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd.inputs import random_dout, random_qkv, sample_rows
from oracle import ref
from tests.parity import say, widen

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE, TOL_G = 1e-2, 1e-3, 1e-2


def fwd_check(name, q, k, v, causal, scale, rows=None):
    say("case %s: B,H,Lq,Lk,d=%s causal=%d fp16" % (name, tuple(q.shape[:3]) + (k.shape[2], q.shape[3]), causal))
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
    o_ref, lse_ref = ref.attention_f64(widen(q), widen(k), widen(v), scale, causal, rows=rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    eo, el = float(np.max(np.abs(o - o_ref))), float(np.max(np.abs(lse - lse_ref)))
    say("  %-40s max|dO|=%.3e  max|dLSE|=%.3e" % (name, eo, el))
    assert eo <= TOL_O and el <= TOL_LSE, name


SHAPES = [(1, 1, 1, 1, 64), (1, 2, 129, 129, 64), (2, 1, 257, 255, 128), (1, 1, 300, 1, 128),
          (1, 1, 1, 300, 64), (1, 2, 500, 777, 128), (1, 2, 129, 300, 32), (1, 1, 200, 300, 256),
          (1, 2, 200, 300, 96)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_forward_parity(shape, causal):
    B, H, Lq, Lk, d = shape
    q, k, v = random_qkv(B, H, Lq, Lk, d, "fp16", seed=sum(shape) + 9 * causal)
    fwd_check("fp16 %s" % (shape,), q, k, v, causal, float(np.float32(1 / np.sqrt(d))))


def test_f16_forward_peaky():
    q, k, v = random_qkv(1, 2, 700, 900, 128, "fp16", seed=61, q_mult=4.0)
    fwd_check("fp16 peaky", q, k, v, False, float(np.float32(1 / np.sqrt(128))))


def test_f16_forward_headline_shape_sampled():
    """B=2, H=32, N=4096, d=128, causal, fp16; the same 256 sampled rows of every head."""
    q, k, v = random_qkv(2, 32, 4096, 4096, 128, "fp16", seed=3)
    rows = sample_rows(4096, 256, 3000)
    fwd_check("fp16 N=4096 causal", q, k, v, True, float(np.float32(1 / np.sqrt(128))), rows=rows)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 129, 129, 64), (2, 1, 257, 255, 128), (1, 1, 500, 300, 128),
                                   (1, 2, 200, 333, 96), (1, 1, 150, 270, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_f16_backward_parity(shape, causal):
    B, H, Lq, Lk, d = shape
    seed = sum(shape) + 13 * causal
    q, k, v = random_qkv(B, H, Lq, Lk, d, "fp16", seed=seed)
    do = random_dout(B, H, Lq, d, "fp16", seed=seed)
    scale = float(np.float32(1 / np.sqrt(d)))
    tq, tk, tv, tdo = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
    grads = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert all(g.dtype == torch.float16 for g in grads)
    want = ref.attention_bwd_f64(widen(q), widen(k), widen(v), widen(do), scale, causal)
    for label, g, w in zip(("dq", "dk", "dv"), grads, want):
        g = g.double().cpu().numpy()
        bar = TOL_G * max(1.0, float(np.max(np.abs(w))))
        err = float(np.max(np.abs(g - w)))
        say("  fp16 bwd %s %s max|err|=%.3e bar %.3e" % (shape, label, err, bar))
        assert err <= bar, (shape, label)
