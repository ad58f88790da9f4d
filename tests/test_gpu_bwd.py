"""Parity of the HIP backward pass (fa2_bwd, through the C ABI) with the float64 oracle.

The device runs its own forward (fa2_fwd) for o and lse and then fa2_bwd; the
oracle computes dQ, dK, dV from q, k, v and dO alone, by the chain rule through
the attention definition.  Bar (bf16 inputs and outputs): for each gradient G,
max|G_gpu - G_ref| <= 2e-2 * max(1, max|G_ref|) -- the forward's bf16 output bar
scaled to the gradient's magnitude, since every error term (bf16 rounding of
P, dS, O and of the outputs, each 2^-9 relative) is proportional to it.
"""
import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd.inputs import WORKLOADS, random_dout, random_qkv, sample_rows, workload_inputs
from oracle import ref
from tests.parity import say, widen

pytestmark = pytest.mark.gpu

REL_TOL = 2e-2


def gpu_grads(q, k, v, do, causal, scale):
    """CPU bf16 tensors in; (dq, dk, dv) float64 numpy out, via fa2_fwd then fa2_bwd."""
    tq, tk, tv, tdo = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return tuple(t.double().cpu().numpy() for t in (dq, dk, dv))


def compare_grads(name, got, want):
    for label, g, w in zip(("dq", "dk", "dv"), got, want):
        assert np.all(np.isfinite(g)), "%s: non-finite %s" % (name, label)
        scale = max(1.0, float(np.max(np.abs(w)))) if w.size else 1.0
        err = float(np.max(np.abs(g - w))) if w.size else 0.0
        say("  %-40s %s max|err|=%.3e  (max|ref|=%.3e, bar %.3e)" % (name, label, err, scale, REL_TOL * scale))
        assert err <= REL_TOL * scale, "%s: %s error %.3e > %.3e" % (name, label, err, REL_TOL * scale)


def check_full(name, q, k, v, do, causal, scale):
    say("case %s: B,H,Lq,Lk,d=%s causal=%d" % (name, tuple(q.shape[:3]) + (k.shape[2], q.shape[3]), causal))
    got = gpu_grads(q, k, v, do, causal, scale)
    want = ref.attention_bwd_f64(widen(q), widen(k), widen(v), widen(do), scale, causal)
    compare_grads(name, got, want)


SHAPES = [
    # B, H, Lq, Lk, d
    (1, 1, 1, 1, 64),
    (1, 1, 1, 300, 64),
    (1, 1, 300, 1, 128),
    (1, 2, 33, 47, 64),
    (2, 1, 129, 129, 128),
    (1, 2, 257, 255, 128),
    (1, 1, 128, 128, 64),
    (1, 1, 200, 500, 128),
    (1, 1, 500, 200, 64),
    (2, 2, 384, 384, 128),
    (1, 2, 129, 129, 32),
    (1, 1, 300, 200, 32),
    (1, 2, 129, 129, 96),
    (2, 1, 300, 511, 96),
    (1, 1, 1, 300, 96),
    (1, 2, 129, 129, 256),
    (1, 1, 300, 200, 256),
    (2, 1, 65, 333, 256),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_parity_ragged(shape, causal):
    B, H, Lq, Lk, d = shape
    seed = sum(shape) + 11 * causal
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=seed)
    do = random_dout(B, H, Lq, d, "bf16", seed=seed)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))
    check_full("bwd %s" % (shape,), q, k, v, do, causal, scale)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_bwd_loop_trip_counts(n, d, causal):
    """The dK/dV loop runs three steps per trip (ceil(Lq / 64) + 1 steps in all)
    and the dQ loop two (ceil(Lk / 64) steps): lengths 64 n - 5 for n = 1..6 give
    every remainder of both, each with a ragged last tile."""
    L = 64 * n - 5
    seed = 500 + 10 * n + d + causal
    q, k, v = random_qkv(1, 2, L, L, d, "bf16", seed=seed)
    do = random_dout(1, 2, L, d, "bf16", seed=seed)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))
    check_full("bwd trips n=%d d=%d" % (n, d), q, k, v, do, causal, scale)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_parity_large_score_range(causal):
    """Q x 4: peaky rows, probabilities near 0 and 1."""
    q, k, v = random_qkv(1, 2, 300, 450, 128, "bf16", seed=77, q_mult=4.0)
    do = random_dout(1, 2, 300, 128, "bf16", seed=77)
    check_full("bwd peaky", q, k, v, do, causal, float(np.float32(1 / np.sqrt(128))))


@pytest.mark.parametrize("name", ["B4_H16_L2048_d64_bf16", "B4_H16_L2048_d64_bf16_causal",
                                  "B2_H32_L4096_d128_bf16_causal", "B3_H8_Lq1000_Lk7777_d128_bf16_q4"])
def test_bwd_parity_workload(name):
    """Full-size workload on the device; the oracle checks 2 heads, on 256 sampled
    query rows (dq) and 256 sampled keys (dk, dv) each."""
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    do = random_dout(w.B, w.H, w.Lq, w.d, "bf16", seed=w.seed)
    say("case %s (bwd)" % name)
    dq, dk, dv = gpu_grads(q, k, v, do, w.causal, w.scale)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    for b, h in heads:
        rows = sample_rows(w.Lq, 256, w.seed + 2000 + b * w.H + h)
        keys = sample_rows(w.Lk, 256, w.seed + 3000 + b * w.H + h)
        sl = (slice(b, b + 1), slice(h, h + 1))
        want = ref.attention_bwd_f64(widen(q[sl]), widen(k[sl]), widen(v[sl]), widen(do[sl]), w.scale, w.causal,
                                     rows=rows, keys=keys)
        got = (dq[b, h, rows][None, None], dk[b, h, keys][None, None], dv[b, h, keys][None, None])
        compare_grads("%s head (%d,%d)" % (name, b, h), got, want)


def test_bwd_parity_d96_long():
    """d = 96 at N=4096 (B=2, H=16, causal); 2 heads, 256 sampled rows and keys each."""
    B, H, L, d = 2, 16, 4096, 96
    q, k, v = random_qkv(B, H, L, L, d, "bf16", seed=963)
    do = random_dout(B, H, L, d, "bf16", seed=963)
    scale = float(np.float32(1 / np.sqrt(d)))
    say("case d96 long (bwd)")
    dq, dk, dv = gpu_grads(q, k, v, do, True, scale)
    for b, h in [(0, 0), (B - 1, H - 1)]:
        rows = sample_rows(L, 256, 964 + b * H + h)
        keys = sample_rows(L, 256, 965 + b * H + h)
        sl = (slice(b, b + 1), slice(h, h + 1))
        want = ref.attention_bwd_f64(widen(q[sl]), widen(k[sl]), widen(v[sl]), widen(do[sl]), scale, True,
                                     rows=rows, keys=keys)
        got = (dq[b, h, rows][None, None], dk[b, h, keys][None, None], dv[b, h, keys][None, None])
        compare_grads("d96 long head (%d,%d)" % (b, h), got, want)


def test_bwd_parity_d256_long():
    """d = 256 at N=2048 (B=1, H=8, causal); 2 heads, 256 sampled rows and keys each."""
    B, H, L, d = 1, 8, 2048, 256
    q, k, v = random_qkv(B, H, L, L, d, "bf16", seed=2561)
    do = random_dout(B, H, L, d, "bf16", seed=2561)
    scale = float(np.float32(1 / np.sqrt(d)))
    say("case d256 long (bwd)")
    dq, dk, dv = gpu_grads(q, k, v, do, True, scale)
    for b, h in [(0, 0), (B - 1, H - 1)]:
        rows = sample_rows(L, 256, 2562 + b * H + h)
        keys = sample_rows(L, 256, 2563 + b * H + h)
        sl = (slice(b, b + 1), slice(h, h + 1))
        want = ref.attention_bwd_f64(widen(q[sl]), widen(k[sl]), widen(v[sl]), widen(do[sl]), scale, True,
                                     rows=rows, keys=keys)
        got = (dq[b, h, rows][None, None], dk[b, h, keys][None, None], dv[b, h, keys][None, None])
        compare_grads("d256 long head (%d,%d)" % (b, h), got, want)


def test_bwd_closed_forms():
    """Lk = 1: O = V0 whatever Q and K are -> dQ = dK = 0 and dV0 = sum of dO.

    dS = P (dP - D) with dP = dO.v0 (matrix core) and D = dO.o (prep kernel) is
    the difference of two fp32 sums of the same 128 products in different
    orders, so dQ and dK are 0 up to fp32 rounding: |dP| <= ~30 here, 128
    roundings of 2^-24 relative each give a bound near 1e-4."""
    q, k, v = random_qkv(1, 2, 150, 1, 128, "bf16", seed=12)
    do = random_dout(1, 2, 150, 128, "bf16", seed=12)
    for causal in (False, True):
        dq, dk, dv = gpu_grads(q, k, v, do, causal, 0.125)
        assert np.max(np.abs(dq)) <= 1e-4 and np.max(np.abs(dk)) <= 1e-4
        want = widen(do).sum(axis=2)
        assert np.max(np.abs(dv[:, :, 0] - want)) <= REL_TOL * max(1.0, np.max(np.abs(want)))


def test_bwd_unseen_keys_get_zero():
    """Causal with Lk > Lq: keys after the last query are seen by no row -> dK = dV = 0."""
    q, k, v = random_qkv(1, 1, 100, 400, 64, "bf16", seed=13)
    do = random_dout(1, 1, 100, 64, "bf16", seed=13)
    tq, tk, tv, tdo = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, causal=True)
    dk = torch.full_like(tk, float("nan"))
    dv = torch.full_like(tv, float("nan"))
    fa.backward(tq, tk, tv, o, lse, tdo, causal=True, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
    assert (dk[:, :, 100:] == 0).all() and (dv[:, :, 100:] == 0).all()


def test_bwd_bitwise_repeatable():
    q, k, v = (t.cuda() for t in random_qkv(1, 3, 700, 900, 128, "bf16", seed=14))
    do = random_dout(1, 3, 700, 128, "bf16", seed=14).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    g1 = fa.backward(q, k, v, o, lse, do, causal=True)
    g2 = fa.backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


def test_bwd_error_paths_on_device():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1, 8, device="cuda")
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FA2Error) as e:
        fa.backward(q, q, q, q, lse, q, workspace=small)
    assert e.value.status == 8
