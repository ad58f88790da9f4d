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


# ------------------------------------------------ fp16 twins of the other paths
def _cmp(name, o, lse, o_ref, lse_ref, bar_o=TOL_O):
    o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), name
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse[~empty] - lse_ref[~empty]))) if (~empty).any() else 0.0
    say("  %-40s max|dO|=%.3e (bar %.2e)  max|dLSE|=%.3e" % (name, eo, bar_o, el))
    assert eo <= bar_o and el <= TOL_LSE, name


def _grads_cmp(name, got, want, floor=1.0):
    for label, g, w in zip(("dq", "dk", "dv"), got, want):
        assert g.dtype == torch.float16
        err = float(np.max(np.abs(g.double().cpu().numpy() - w)))
        bar = TOL_G * max(floor, float(np.max(np.abs(w))))
        say("  %s %s max|err|=%.3e bar %.3e" % (name, label, err, bar))
        assert err <= bar, (name, label)


@pytest.mark.parametrize("case", [(1, 2, 300, 400, 128, 50, 0), (2, 1, 257, 255, 64, 31, 7),
                                  (1, 1, 400, 100, 96, 10, 0)], ids=lambda c: "x".join(map(str, c)))
def test_f16_window_forward_and_backward(case):
    B, H, Lq, Lk, d, wl, wr = case
    q, k, v = random_qkv(B, H, Lq, Lk, d, "fp16", seed=sum(case))
    do = random_dout(B, H, Lq, d, "fp16", seed=sum(case))
    scale = float(np.float32(1 / np.sqrt(d)))
    say("case fp16 window %s" % (case,))
    tq, tk, tv, tdo = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, scale=scale, window=(wl, wr))
    grads = fa.backward(tq, tk, tv, o, lse, tdo, scale=scale, window=(wl, wr))
    torch.cuda.synchronize()
    o_ref, l_ref = ref.attention_window_f64(widen(q), widen(k), widen(v), scale, wl, wr)
    _cmp("fp16 window", o, lse, o_ref, l_ref)
    _grads_cmp("fp16 window bwd", grads,
               ref.attention_bwd_f64(widen(q), widen(k), widen(v), widen(do), scale, False, window=(wl, wr)))


@pytest.mark.parametrize("case", [(1, 2, 300, 300, 128, True, 0.2), (2, 1, 200, 333, 64, False, 0.5)],
                         ids=lambda c: "x".join(map(str, c)))
def test_f16_dropout_forward_and_backward(case):
    B, H, Lq, Lk, d, causal, p = case
    q, k, v = random_qkv(B, H, Lq, Lk, d, "fp16", seed=Lq + Lk)
    do = random_dout(B, H, Lq, d, "fp16", seed=Lq + Lk)
    scale = float(np.float32(1 / np.sqrt(d)))
    seed, offset, t = 0xF16, 9, ref.dropout_threshold(p)
    say("case fp16 dropout %s" % (case,))
    tq, tk, tv, tdo = (x.cuda() for x in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale, dropout=(p, seed, offset))
    grads = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale, dropout=(p, seed, offset))
    torch.cuda.synchronize()
    o_ref, l_ref, *g_ref = ref.attention_dropout_f64(widen(q), widen(k), widen(v), scale, causal, seed, offset, t,
                                                      dout=widen(do))
    _cmp("fp16 dropout", o, lse, o_ref, l_ref, bar_o=TOL_O * 256.0 / t)
    _grads_cmp("fp16 dropout bwd", grads, g_ref, floor=256.0 / t)


@pytest.mark.parametrize("shape", [(1, 2, 300, 5000, 128), (2, 3, 1, 3000, 64), (1, 2, 3, 777, 96)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
def test_f16_splitkv(shape, causal):
    """fp16 split-KV: the MFMA partial kernel (Lq > 4) or the decoding kernel, then the fp16 merge."""
    B, H, Lq, Lk, d = shape
    q, k, v = random_qkv(B, H, Lq, Lk, d, "fp16", seed=sum(shape) + causal)
    scale = float(np.float32(1 / np.sqrt(d)))
    for splits in (3, 0):
        say("case fp16 split-KV %s causal=%d S=%d" % (shape, causal, splits))
        o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, num_splits=splits)
        torch.cuda.synchronize()
        assert o.dtype == torch.float16
        o_ref, l_ref = ref.attention_f64(widen(q), widen(k), widen(v), scale, causal)
        _cmp("fp16 split S=%d" % splits, o, lse, o_ref, l_ref)


def test_f16_merge_partials():
    B, H, Lq, Lk, d = 1, 2, 50, 700, 64
    q, k, v = (widen(t) for t in random_qkv(B, H, Lq, Lk, d, "fp16", seed=52))
    bounds = [(0, 200), (200, 201), (201, 700)]
    parts = [ref.attention_f64(q, k[:, :, a:b], v[:, :, a:b], 0.125, False) for a, b in bounds]
    o_parts = np.stack([p[0] for p in parts]).astype(np.float32)
    l_parts = np.stack([p[1] for p in parts]).astype(np.float32)
    o_ref, l_ref = ref.merge_partials(o_parts, l_parts)
    o, lse = fa.merge_partials(torch.from_numpy(o_parts).cuda(), torch.from_numpy(l_parts).cuda(),
                               dtype=torch.float16)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    eo = float(np.max(np.abs(o.double().cpu().numpy() - o_ref)))
    el = float(np.max(np.abs(lse.double().cpu().numpy() - l_ref)))
    say("  fp16 merge max|dO|=%.3e max|dLSE|=%.3e" % (eo, el))
    assert eo <= 2 ** -10 * max(1.0, float(np.abs(o_ref).max())) and el <= 1e-5   # one fp16 ulp
