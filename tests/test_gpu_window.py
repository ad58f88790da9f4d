"""Parity of the sliding-window forward (fa2_fwd_window, through the C ABI) with
the float64 window oracle.  Bars as fa2_fwd's bf16 bars (max|O| 2e-2, max|LSE|
1e-3); rows that see no key must give O = 0 and LSE = -inf exactly."""
import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd.inputs import random_qkv, sample_rows
from oracle import ref
from tests.parity import TOL, say, widen

pytestmark = pytest.mark.gpu


def run_window(q, k, v, scale, wl, wr):
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), scale=scale, window=(wl, wr))
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def check(name, q, k, v, scale, wl, wr, rows=None):
    say("case %s: B,H,Lq,Lk,d=%s window=(%d,%d)" % (name, tuple(q.shape[:3]) + (k.shape[2], q.shape[3]), wl, wr))
    o, lse = run_window(q, k, v, scale, wl, wr)
    o_ref, lse_ref = ref.attention_window_f64(widen(q), widen(k), widen(v), scale, wl, wr, rows=rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), "%s: empty rows differ" % name
    assert np.all(o[empty] == 0), "%s: empty rows must have O = 0" % name
    eo = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    el = float(np.max(np.abs(lse[~empty] - lse_ref[~empty]))) if (~empty).any() else 0.0
    say("  %-40s max|dO|=%.3e  max|dLSE|=%.3e  empty rows %d" % (name, eo, el, int(empty.sum())))
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"], name


CASES = [
    # B, H, Lq, Lk, d, wl, wr
    (1, 1, 1, 1, 64, 0, 0),
    (1, 2, 300, 300, 64, 16, 0),
    (1, 1, 500, 500, 128, 100, 0),
    (2, 2, 257, 255, 128, 31, 7),
    (1, 1, 200, 600, 64, 64, 64),
    (1, 1, 400, 100, 64, 10, 0),        # rows >= 111 see no key
    (1, 1, 333, 333, 128, 0, 0),
    (1, 2, 700, 900, 128, -1, 50),
    (1, 1, 640, 640, 64, 127, -1),
    (2, 1, 384, 384, 128, 200, 200),
    (1, 1, 129, 1000, 128, 5, 900),
    (1, 2, 300, 300, 32, 20, 0),
    (1, 1, 300, 400, 256, 50, 10),
    (1, 2, 300, 500, 96, 40, 5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_window_parity(case):
    B, H, Lq, Lk, d, wl, wr = case
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=sum(case) + 3)
    check("window", q, k, v, float(np.float32(1 / np.sqrt(d))), wl, wr)


def test_window_peaky():
    q, k, v = random_qkv(1, 2, 600, 600, 128, "bf16", seed=31, q_mult=4.0)
    check("window peaky", q, k, v, float(np.float32(1 / np.sqrt(128))), 150, 0)


def test_window_long_sequence_sampled():
    """N=8192, d=128, causal window of 1024 keys; 512 sampled rows per head."""
    q, k, v = random_qkv(1, 4, 8192, 8192, 128, "bf16", seed=40)
    rows = sample_rows(8192, 512, 41, forced=(0, 1, 63, 64, 127, 128, 1023, 1024, 1025))
    check("window long", q, k, v, float(np.float32(1 / np.sqrt(128))), 1023, 0, rows=rows)


@pytest.mark.parametrize("causal", [False, True])
def test_window_matches_plain_forward(causal):
    """(-1, -1) and (-1, 0) give fa2_fwd's full and causal results."""
    q, k, v = (t.cuda() for t in random_qkv(1, 3, 500, 500, 128, "bf16", seed=42))
    o1, l1 = fa.forward(q, k, v, causal=causal)
    o2, l2 = fa.forward(q, k, v, window=(-1, 0 if causal else -1))
    torch.cuda.synchronize()
    assert torch.max(torch.abs(o1.float() - o2.float())).item() <= 1e-2
    assert torch.max(torch.abs(l1 - l2)).item() <= 1e-5


# ------------------------------------------------------------------ backward
BWD_CASES = [
    # B, H, Lq, Lk, d, wl, wr
    (1, 2, 300, 300, 64, 16, 0),
    (1, 1, 500, 500, 128, 100, 0),
    (2, 1, 257, 255, 128, 31, 7),
    (1, 1, 200, 600, 64, 64, 64),
    (1, 1, 400, 100, 64, 10, 0),        # rows >= 111 see no key; keys seen by few rows
    (1, 1, 333, 333, 128, 0, 0),
    (1, 2, 384, 512, 128, -1, 50),
    (1, 1, 640, 640, 64, 127, -1),
    (1, 2, 300, 300, 32, 20, 3),
    (1, 2, 300, 400, 96, 50, 0),
    (1, 1, 300, 400, 256, 70, 10),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c)))
def test_window_backward_parity(case):
    from flashattention_forward_fwd_amd.inputs import random_dout
    from tests.test_gpu_bwd import compare_grads
    B, H, Lq, Lk, d, wl, wr = case
    seed = sum(case) + 5
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=seed)
    do = random_dout(B, H, Lq, d, "bf16", seed=seed)
    scale = float(np.float32(1 / np.sqrt(d)))
    say("case window bwd %s" % (case,))
    tq, tk, tv, tdo = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, scale=scale, window=(wl, wr))
    grads = fa.backward(tq, tk, tv, o, lse, tdo, scale=scale, window=(wl, wr))
    torch.cuda.synchronize()
    got = tuple(g.double().cpu().numpy() for g in grads)
    want = ref.attention_bwd_f64(widen(q), widen(k), widen(v), widen(do), scale, False, window=(wl, wr))
    compare_grads("window bwd %s" % (case,), got, want)


def test_window_backward_causal_matches_fa2_bwd():
    """(-1, 0) through fa2_bwd_window gives fa2_bwd's causal gradients bit for bit."""
    from flashattention_forward_fwd_amd.inputs import random_dout
    q, k, v = (t.cuda() for t in random_qkv(1, 2, 700, 700, 128, "bf16", seed=50))
    do = random_dout(1, 2, 700, 128, "bf16", seed=50).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    g1 = fa.backward(q, k, v, o, lse, do, causal=True)
    g2 = fa.backward(q, k, v, o, lse, do, window=(-1, 0))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
