"""Parity of attention with dropout (fa2_fwd_dropout, through the C ABI) with the
float64 dropout oracle.

The keep mask is integer work decided by the generator alone, so it is checked
bit-exactly: with V = I (Lk <= d) the output row i is row i of A = P * Z * 256 / t,
and its zeros must be exactly the dropped or masked pairs.  Values: the bf16
bars of fa2_fwd scaled by the keep scale 256 / t (every kept probability, and so
every rounding error carried by O, grows by that factor): max|dO| <= 2e-2 * 256 / t,
max|dLSE| <= 1e-3 (the LSE is the one without dropout)."""
import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd.inputs import random_dout, random_qkv
from oracle import ref
from tests.parity import TOL, say, widen

pytestmark = pytest.mark.gpu


def run_dropout(q, k, v, causal, scale, p, seed, offset):
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, dropout=(p, seed, offset))
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def check(name, q, k, v, causal, scale, p, seed, offset):
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    t = ref.dropout_threshold(p)
    say("case %s: B,H,Lq,Lk,d=%s causal=%d p=%g (t=%d) seed=%#x offset=%d"
        % (name, (B, H, Lq, Lk, d), causal, p, t, seed, offset))
    o, lse = run_dropout(q, k, v, causal, scale, p, seed, offset)
    o_ref, lse_ref = ref.attention_dropout_f64(widen(q), widen(k), widen(v), scale, causal, seed, offset, t)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), name
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse - lse_ref)))
    bar = TOL["bf16"]["o"] * 256.0 / t
    say("  %-40s max|dO|=%.3e (bar %.2e)  max|dLSE|=%.3e" % (name, eo, bar, el))
    assert eo <= bar and el <= TOL["bf16"]["lse"], name


CASES = [
    # B, H, Lq, Lk, d, causal, p
    (1, 2, 300, 300, 128, True, 0.1),
    (2, 3, 200, 333, 64, False, 0.25),
    (1, 1, 257, 513, 128, False, 0.5),
    (1, 2, 300, 300, 32, True, 0.2),
    (1, 1, 300, 400, 256, True, 0.15),
    (1, 2, 300, 400, 96, False, 0.2),
    (1, 1, 1, 1, 64, False, 0.3),
    (1, 1, 130, 70, 128, True, 0.9),
    (2, 2, 129, 1000, 128, False, 0.05),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_dropout_forward_parity(case):
    B, H, Lq, Lk, d, causal, p = case
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=Lq + Lk + d)
    check("dropout", q, k, v, causal, float(np.float32(1 / np.sqrt(d))), p, 0x5EED0000 + Lq, Lk)


def test_dropout_peaky_rows():
    q, k, v = random_qkv(1, 2, 400, 400, 128, "bf16", seed=77, q_mult=4.0)
    check("dropout peaky", q, k, v, True, float(np.float32(1 / np.sqrt(128))), 0.2, 12345, 3)


@pytest.mark.parametrize("d,Lk,causal", [(128, 128, False), (128, 100, True), (256, 250, False), (64, 64, True),
                                         (32, 32, False), (96, 96, True)])
def test_dropout_mask_exact(d, Lk, causal):
    """V = I: the nonzero pattern of O[..., :Lk] is the keep mask (and the causal
    mask), bit for bit, for a seed using both key words and a nonzero offset."""
    B, H, Lq = 2, 3, 300
    q, k, _ = random_qkv(B, H, Lq, Lk, d, "bf16", seed=d + Lk)
    v = torch.zeros(B, H, Lk, d, dtype=torch.bfloat16)
    v[:, :, torch.arange(Lk), torch.arange(Lk)] = 1.0
    p, seed, offset = 0.3, 0x0123456789ABCDEF, 0xDEADBEEF
    t = ref.dropout_threshold(p)
    say("case mask_exact d=%d Lk=%d causal=%d" % (d, Lk, causal))
    o, _ = run_dropout(q, k, v, causal, float(np.float32(1 / np.sqrt(d))), p, seed, offset)
    want = ref.dropout_mask(B, H, Lq, Lk, seed, offset, t)
    if causal:
        want &= np.tril(np.ones((Lq, Lk), dtype=bool))
    got = o[..., :Lk] != 0
    say("  kept %d of %d, mismatches %d" % (int(want.sum()), want.size, int((got != want).sum())))
    assert np.array_equal(got, want)
    assert np.all(o[..., Lk:] == 0)


def test_dropout_zero_rate_is_plain_forward():
    q, k, v = (x.cuda() for x in random_qkv(1, 2, 300, 300, 128, "bf16", seed=5))
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k, v, causal=True, dropout=(0.0, 99, 1))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_dropout_seed_and_offset_select_the_mask():
    q, k, v = (x.cuda() for x in random_qkv(1, 2, 200, 200, 64, "bf16", seed=6))
    a, la = fa.forward(q, k, v, dropout=(0.2, 7, 0))
    b, _ = fa.forward(q, k, v, dropout=(0.2, 7, 0))
    c, _ = fa.forward(q, k, v, dropout=(0.2, 7, 1))
    e, _ = fa.forward(q, k, v, dropout=(0.2, 7 + (1 << 32), 0))
    plain, lp = fa.forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)                     # deterministic
    assert not torch.equal(a, c) and not torch.equal(a, e)
    assert torch.equal(la, lp)                   # the LSE ignores dropout


def test_dropout_headline_shape_first_head():
    """B=2, H=32, N=4096, d=128, causal, p=0.1: head (0, 0) (generator counter word
    b*H + h = 0) against the oracle run on that head alone; every head's LSE
    against fa2_fwd's."""
    B, H, L, d = 2, 32, 4096, 128
    q, k, v = random_qkv(B, H, L, L, d, "bf16", seed=2024)
    scale = float(np.float32(1 / np.sqrt(d)))
    p, seed, offset = 0.1, 0xABCDEF, 17
    t = ref.dropout_threshold(p)
    say("case dropout headline B=2 H=32 N=4096 d=128 causal p=0.1")
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.forward(qc, kc, vc, causal=True, scale=scale, dropout=(p, seed, offset))
    _, lse_plain = fa.forward(qc, kc, vc, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse_plain)
    o0 = o[0, 0].double().cpu().numpy()
    o_ref, l_ref = ref.attention_dropout_f64(widen(q[:1, :1]), widen(k[:1, :1]), widen(v[:1, :1]), scale, True,
                                             seed, offset, t)
    eo = float(np.max(np.abs(o0 - o_ref[0, 0])))
    el = float(np.max(np.abs(lse[0, 0].double().cpu().numpy() - l_ref[0, 0])))
    bar = TOL["bf16"]["o"] * 256.0 / t
    say("  head (0,0): max|dO|=%.3e (bar %.2e) max|dLSE|=%.3e" % (eo, bar, el))
    assert eo <= bar and el <= TOL["bf16"]["lse"]


# ------------------------------------------------------------------ backward
def grad_bar(g_ref, t):
    """Backward bar with dropout: 2e-2 * max(256 / t, max|G_ref|) -- the bf16 bar of
    the plain backward with its O(1) floor raised by the keep scale, the factor on
    every kept probability and on dP."""
    return 2e-2 * max(256.0 / t, float(np.abs(g_ref).max()))


def run_dropout_bwd(q, k, v, do, causal, scale, p, seed, offset):
    tq, tk, tv, tdo = (x.cuda() for x in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale, dropout=(p, seed, offset))
    grads = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale, dropout=(p, seed, offset))
    torch.cuda.synchronize()
    return [g.double().cpu().numpy() for g in grads]


def check_bwd(name, q, k, v, do, causal, scale, p, seed, offset):
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    t = ref.dropout_threshold(p)
    say("case %s: B,H,Lq,Lk,d=%s causal=%d p=%g (t=%d)" % (name, (B, H, Lq, Lk, d), causal, p, t))
    got = run_dropout_bwd(q, k, v, do, causal, scale, p, seed, offset)
    want = ref.attention_dropout_f64(widen(q), widen(k), widen(v), scale, causal, seed, offset, t, dout=widen(do))[2:]
    for gname, g, w in zip(("dq", "dk", "dv"), got, want):
        assert np.all(np.isfinite(g)), "%s %s: non-finite" % (name, gname)
        err = float(np.max(np.abs(g - w)))
        bar = grad_bar(w, t)
        say("  %-32s %s max|err|=%.3e (bar %.3e, max|G|=%.3e)" % (name, gname, err, bar, float(np.abs(w).max())))
        assert err <= bar, "%s %s" % (name, gname)


BWD_CASES = [
    # B, H, Lq, Lk, d, causal, p
    (1, 2, 300, 300, 128, True, 0.1),
    (2, 3, 200, 333, 64, False, 0.25),
    (1, 1, 257, 513, 128, False, 0.5),
    (1, 2, 300, 300, 32, True, 0.2),
    (1, 1, 130, 70, 128, True, 0.9),
    (1, 1, 1, 1, 64, False, 0.3),
    (2, 2, 129, 1000, 128, False, 0.05),
    (1, 1, 640, 640, 128, True, 0.3),
    (1, 1, 333, 129, 64, True, 0.6),
    (1, 2, 300, 257, 96, False, 0.25),
    (1, 1, 200, 300, 256, True, 0.2),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c)))
def test_dropout_backward_parity(case):
    B, H, Lq, Lk, d, causal, p = case
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=Lq + 2 * Lk + d)
    do = random_dout(B, H, Lq, d, "bf16", seed=Lq + 2 * Lk + d)
    check_bwd("dropout bwd", q, k, v, do, causal, float(np.float32(1 / np.sqrt(d))), p, 0xC0FFEE + Lk, Lq)


@pytest.mark.parametrize("case", [
    # Lq, d, p, inputs seed, dropout seed, offset
    (65, 64, 0.1, 2015, 5487277651644988878, 72267039),
    (200, 128, 0.3, 7, 0xABCDEF, 5),
    (129, 32, 0.5, 8, 0x13579BDF, 77),
], ids=lambda c: "Lq%d-d%d-p%g" % c[:3])
def test_dropout_backward_single_key(case):
    """One key: P = 1 on every row, so dS = P (dP - D) and with it dQ and dK vanish
    exactly.  The backward forms D = rowsum(dO * O) from the forward's stored 16-bit
    O ("FlashAttention 怎么做? online softmax 怎么更新?", section "Recomputation"),
    and under dropout O = V * 256 / t is not a bf16 value, so what the device returns
    here is the rounding of O carried through D -- an error on the scale of
    |dO| |O|, not of the (zero) gradient.  Checked against that quantity in float64:
    the same formulas with D taken from O rounded to bf16 (nearest even)."""
    Lq, d, p, in_seed, seed, offset = case
    q, k, v = random_qkv(1, 1, Lq, 1, d, "bf16", seed=in_seed)
    do = random_dout(1, 1, Lq, d, "bf16", seed=in_seed)
    scale = float(np.float32(1 / np.sqrt(d)))
    t = ref.dropout_threshold(p)
    ks = 256.0 / t
    say("case dropout bwd single key Lq=%d d=%d p=%g" % (Lq, d, p))
    got = run_dropout_bwd(q, k, v, do, False, scale, p, seed, offset)
    exact = ref.attention_dropout_f64(widen(q), widen(k), widen(v), scale, False, seed, offset, t, dout=widen(do))[2:]
    Q, K, V, dO = (widen(x)[0, 0] for x in (q, k, v, do))
    Z = ref.dropout_mask(1, 1, Lq, 1, seed, offset, t)[0, 0].astype(np.float64)
    A = Z * ks                                            # P = 1
    O16 = torch.from_numpy(A @ V).to(torch.bfloat16).double().numpy()
    D = np.sum(dO * O16, axis=1, keepdims=True)
    dS = A / ks * (dO @ V.T * A - D)                     # P (dP - D), dP = dO V^T * Z * ks
    model = (scale * dS @ K, scale * dS.T @ Q)
    for gname, g, e, m in zip(("dq", "dk"), got[:2], exact[:2], model):
        g = g[0, 0]
        err = float(np.max(np.abs(g - m)))
        bar = 5e-2 * float(np.abs(m).max()) + 1e-3
        say("  %s max|G| %.3e (exact %.1e)  max|G - model| %.3e (bar %.3e)" % (
            gname, float(np.abs(g).max()), float(np.abs(e).max()), err, bar))
        assert float(np.abs(e).max()) < 1e-9 and err <= bar, gname


def test_dropout_backward_zero_rate_is_plain_backward():
    q, k, v = (x.cuda() for x in random_qkv(1, 2, 300, 300, 128, "bf16", seed=8))
    do = random_dout(1, 2, 300, 128, "bf16", seed=8).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    g1 = fa.backward(q, k, v, o, lse, do, causal=True)
    g2 = fa.backward(q, k, v, o, lse, do, causal=True, dropout=(0.0, 5, 5))
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,Lq,causal", [(128, 128, False), (128, 100, True), (64, 64, False), (32, 32, True),
                                         (96, 96, False), (256, 200, True)])
def test_dropout_backward_mask_exact(d, Lq, causal):
    """dout = I (Lq <= d): dv[j, i] = (256 / t) P[i, j] Z[i, j], so the nonzero
    pattern of dv[..., :Lq] is the transposed keep mask (and the causal mask) bit
    for bit -- the mask as the key-per-lane kernel draws it."""
    B, H, Lk = 2, 3, 300
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=d + Lq + 1)
    do = torch.zeros(B, H, Lq, d, dtype=torch.bfloat16)
    do[:, :, torch.arange(Lq), torch.arange(Lq)] = 1.0
    p, seed, offset = 0.3, 0xFEDCBA9876543210, 42
    t = ref.dropout_threshold(p)
    say("case bwd mask_exact d=%d Lq=%d causal=%d" % (d, Lq, causal))
    _, _, dv = run_dropout_bwd(q, k, v, do, causal, float(np.float32(1 / np.sqrt(d))), p, seed, offset)
    want = ref.dropout_mask(B, H, Lq, Lk, seed, offset, t)
    if causal:
        want &= np.tril(np.ones((Lq, Lk), dtype=bool))
    got = np.swapaxes(dv[..., :Lq], -1, -2) != 0
    say("  kept %d of %d, mismatches %d" % (int(want.sum()), want.size, int((got != want).sum())))
    assert np.array_equal(got, want)


def test_dropout_backward_headline_shape_first_head():
    """B=2, H=32, N=4096, d=128, causal, p=0.1: the gradients of head (0, 0)
    against the oracle run on that head alone."""
    B, H, L, d = 2, 32, 4096, 128
    q, k, v = random_qkv(B, H, L, L, d, "bf16", seed=2025)
    do = random_dout(B, H, L, d, "bf16", seed=2025)
    scale = float(np.float32(1 / np.sqrt(d)))
    p, seed, offset = 0.1, 0x1234, 99
    t = ref.dropout_threshold(p)
    say("case dropout backward headline B=2 H=32 N=4096 d=128 causal p=0.1")
    got = run_dropout_bwd(q, k, v, do, True, scale, p, seed, offset)
    want = ref.attention_dropout_f64(widen(q[:1, :1]), widen(k[:1, :1]), widen(v[:1, :1]), scale, True, seed,
                                     offset, t, dout=widen(do[:1, :1]))[2:]
    for gname, g, w in zip(("dq", "dk", "dv"), got, want):
        err = float(np.max(np.abs(g[0, 0] - w[0, 0])))
        bar = grad_bar(w, t)
        say("  head (0,0) %s max|err|=%.3e (bar %.3e)" % (gname, err, bar))
        assert err <= bar, gname
