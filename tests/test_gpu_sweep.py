"""A seeded random sweep of the 16-bit entry points against the float64 oracles.

Each case draws a shape (B, H <= 3; Lq, Lk up to a few hundred, with a few very
short ones), a head dimension, bf16 or fp16, and one of the forward variants
(causal, full, split-KV with 2-7 ranges or the automatic count, decoding rows,
sliding window, dropout) or a backward variant (causal, full, window, dropout).
Bars as the dedicated tests: O 2e-2 (bf16) / 1e-2 (fp16), LSE 1e-3; gradients
2e-2 / 1e-2 times max(1, max|G_ref|); dropout raises the O(1) floors by the keep
scale 256 / t.  dQ and dK also get the amount D = rowsum(dO * O) carries from the
forward's 16-bit O (modelled in float64), which is not on the gradient's scale: it is
what remains where dS vanishes, e.g. one visible key under dropout.  Rows that see no key (window) must give O = 0 and LSE = -inf."""
import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd.inputs import random_dout, random_qkv
from oracle import ref
from tests.parity import say, widen

pytestmark = pytest.mark.gpu

O_BAR = {"bf16": 2e-2, "fp16": 1e-2}
LSE_BAR = 1e-3
DIMS = (32, 64, 96, 128, 256)


def _draw_len(rng):
    r = rng.random()
    if r < 0.1:
        return int(rng.integers(1, 5))
    if r < 0.2:
        return int(rng.choice([63, 64, 65, 127, 128, 129, 255, 256, 257]))
    return int(rng.integers(5, 700))


def _forward_cases(n, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = ["causal", "full", "split", "decode", "window", "dropout"][i % 6]
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        d = int(rng.choice(DIMS))
        Lq, Lk = _draw_len(rng), _draw_len(rng)
        if variant == "decode":
            Lq, Lk = int(rng.integers(1, 5)), int(rng.integers(200, 3000))
        if variant == "dropout":                      # the dropout oracle holds every P
            Lq, Lk = min(Lq, 400), min(Lk, 400)
        extra = {}
        if variant in ("split", "decode"):
            extra["splits"] = int(rng.choice([0, 2, 3, 5, 7]))
            extra["causal"] = bool(rng.random() < 0.5)
        elif variant == "window":
            extra["wl"] = int(rng.choice([-1, 0, int(rng.integers(1, 300))]))
            extra["wr"] = int(rng.choice([-1, 0, int(rng.integers(1, 300))]))
        elif variant == "dropout":
            extra["p"] = float(rng.choice([0.1, 0.3, 0.5, 0.8]))
            extra["seed"] = int(rng.integers(0, 2**63))
            extra["offset"] = int(rng.integers(0, 2**31))
            extra["causal"] = bool(rng.random() < 0.5)
        dtype = "fp16" if rng.random() < 0.35 else "bf16"
        out.append((i, variant, B, H, Lq, Lk, d, dtype, extra))
    return out


def _backward_cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = ["causal", "full", "window", "dropout"][i % 4]
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        d = int(rng.choice(DIMS))
        Lq, Lk = min(_draw_len(rng), 400), min(_draw_len(rng), 400)
        extra = {}
        if variant == "window":
            extra["wl"] = int(rng.choice([-1, int(rng.integers(0, 200))]))
            extra["wr"] = int(rng.choice([-1, 0, int(rng.integers(1, 200))]))
        elif variant == "dropout":
            extra["p"] = float(rng.choice([0.1, 0.3, 0.5]))
            extra["seed"] = int(rng.integers(0, 2**63))
            extra["offset"] = int(rng.integers(0, 2**31))
            extra["causal"] = bool(rng.random() < 0.5)
        dtype = "fp16" if rng.random() < 0.35 else "bf16"
        out.append((i, variant, B, H, Lq, Lk, d, dtype, extra))
    return out


def _case_id(c):
    i, variant, B, H, Lq, Lk, d, dtype, extra = c
    return "%02d-%s-%s-%dx%dx%dx%dx%d" % (i, variant, dtype, B, H, Lq, Lk, d)


def _np(t):
    return t.double().cpu().numpy()


@pytest.mark.parametrize("case", _forward_cases(48), ids=_case_id)
def test_forward_sweep(case):
    i, variant, B, H, Lq, Lk, d, dtype, extra = case
    say("case sweep fwd %s %s" % (_case_id(case), extra))
    q, k, v = random_qkv(B, H, Lq, Lk, d, dtype, seed=1000 + i)
    scale = float(np.float32(1 / np.sqrt(d)))
    tq, tk, tv = q.cuda(), k.cuda(), v.cuda()
    qd, kd, vd = widen(q), widen(k), widen(v)
    bar = O_BAR[dtype]
    if variant in ("causal", "full"):
        causal = variant == "causal"
        o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
        o_ref, l_ref = ref.attention_f64(qd, kd, vd, scale, causal)
    elif variant in ("split", "decode"):
        o, lse = fa.forward(tq, tk, tv, causal=extra["causal"], scale=scale, num_splits=extra["splits"])
        o_ref, l_ref = ref.attention_f64(qd, kd, vd, scale, extra["causal"])
    elif variant == "window":
        o, lse = fa.forward(tq, tk, tv, scale=scale, window=(extra["wl"], extra["wr"]))
        o_ref, l_ref = ref.attention_window_f64(qd, kd, vd, scale, extra["wl"], extra["wr"])
    else:
        t = ref.dropout_threshold(extra["p"])
        drop = (extra["p"], extra["seed"], extra["offset"])
        o, lse = fa.forward(tq, tk, tv, causal=extra["causal"], scale=scale, dropout=drop)
        o_ref, l_ref = ref.attention_dropout_f64(qd, kd, vd, scale, extra["causal"], extra["seed"],
                                                 extra["offset"], t)
        bar *= 256.0 / t
    torch.cuda.synchronize()
    o, lse = _np(o), _np(lse)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), "rows without a visible key differ"
    assert np.all(o[empty] == 0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse[~empty]))
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse[~empty] - l_ref[~empty]))) if (~empty).any() else 0.0
    say("  max|dO|=%.3e (bar %.2e)  max|dLSE|=%.3e  empty rows %d" % (eo, bar, el, int(empty.sum())))
    assert eo <= bar and el <= LSE_BAR


def _d_rounding_term(qd, kd, vd, dod, scale, dtype, causal=False, window=None, drop=None):
    """The part of dQ and dK that D = rowsum(dO * O) carries from the forward's
    16-bit output: with dD = rowsum(dO * (round16(O) - O)) per row, dS moves by
    -P * dD, so dQ by -scale P dD K and dK by -scale (P dD)^T Q (float64, O and P by
    definition; drop = (Z, keep scale) multiplies P by Z * keep scale in O).  Where dS
    vanishes (one visible key: P = 1) this is all that separates the device from the
    exact gradients, an amount on the scale of |dO| |O| rather than of the gradient."""
    B, H, Lq, d = qd.shape
    Lk = kd.shape[2]
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    vis = np.ones((Lq, Lk), dtype=bool)
    if causal:
        vis &= j <= i
    if window is not None:
        wl, wr = window
        if wl >= 0:
            vis &= j >= i - wl
        if wr >= 0:
            vis &= j <= i + wr
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    dq = np.zeros_like(qd)
    dk = np.zeros_like(kd)
    for b in range(B):
        for h in range(H):
            s_ = np.where(vis, scale * qd[b, h] @ kd[b, h].T, -np.inf)
            m = s_.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(s_ - m)
            l = e.sum(axis=1, keepdims=True)
            P = np.divide(e, l, out=np.zeros_like(e), where=l > 0)
            A = P if drop is None else P * drop[0][b, h] * drop[1]
            O = A @ vd[b, h]
            O16 = torch.from_numpy(O).to(tdt).double().numpy()
            dD = np.sum(dod[b, h] * (O16 - O), axis=1, keepdims=True)
            dS = -P * dD
            dq[b, h] = scale * dS @ kd[b, h]
            dk[b, h] = scale * dS.T @ qd[b, h]
    return dq, dk


@pytest.mark.parametrize("case", _backward_cases(16), ids=_case_id)
def test_backward_sweep(case):
    i, variant, B, H, Lq, Lk, d, dtype, extra = case
    say("case sweep bwd %s %s" % (_case_id(case), extra))
    q, k, v = random_qkv(B, H, Lq, Lk, d, dtype, seed=2000 + i)
    do = random_dout(B, H, Lq, d, dtype, seed=2000 + i)
    scale = float(np.float32(1 / np.sqrt(d)))
    tq, tk, tv, tdo = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    qd, kd, vd, dod = widen(q), widen(k), widen(v), widen(do)
    floor = 1.0
    if variant in ("causal", "full"):
        causal = variant == "causal"
        o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
        got = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
        want = ref.attention_bwd_f64(qd, kd, vd, dod, scale, causal)
        term = _d_rounding_term(qd, kd, vd, dod, scale, dtype, causal=causal)
    elif variant == "window":
        w = (extra["wl"], extra["wr"])
        o, lse = fa.forward(tq, tk, tv, scale=scale, window=w)
        got = fa.backward(tq, tk, tv, o, lse, tdo, scale=scale, window=w)
        want = ref.attention_bwd_f64(qd, kd, vd, dod, scale, False, window=w)
        term = _d_rounding_term(qd, kd, vd, dod, scale, dtype, window=w)
    else:
        t = ref.dropout_threshold(extra["p"])
        drop = (extra["p"], extra["seed"], extra["offset"])
        o, lse = fa.forward(tq, tk, tv, causal=extra["causal"], scale=scale, dropout=drop)
        got = fa.backward(tq, tk, tv, o, lse, tdo, causal=extra["causal"], scale=scale, dropout=drop)
        want = ref.attention_dropout_f64(qd, kd, vd, scale, extra["causal"], extra["seed"], extra["offset"], t,
                                         dout=dod)[2:]
        floor = 256.0 / t
        z = ref.dropout_mask(B, H, Lq, Lk, extra["seed"], extra["offset"], t).astype(np.float64)
        term = _d_rounding_term(qd, kd, vd, dod, scale, dtype, causal=extra["causal"], drop=(z, 256.0 / t))
    term = (np.abs(term[0]).max() if term[0].size else 0.0, np.abs(term[1]).max() if term[1].size else 0.0, 0.0)
    torch.cuda.synchronize()
    rel = O_BAR[dtype]
    for name, g, w, dterm in zip(("dq", "dk", "dv"), got, want, term):
        g = _np(g)
        assert np.all(np.isfinite(g)), name
        # the relative bar, plus what D's 16-bit O carries into dQ and dK
        bar = rel * max(floor, float(np.abs(w).max()) if w.size else 0.0) + float(dterm)
        err = float(np.max(np.abs(g - w))) if w.size else 0.0
        say("  %s max|err|=%.3e (bar %.3e, of which D's rounding %.1e)" % (name, err, bar, float(dterm)))
        assert err <= bar, name
