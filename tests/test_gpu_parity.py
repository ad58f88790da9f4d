"""Parity of the HIP forward pass (through the C ABI) with the float64 oracle.

Bars: bf16 inputs -- max|O - O_ref| <= 2e-2 and max|LSE - LSE_ref| <= 1e-3;
fp32 inputs -- both <= 1e-5.  O_ref and LSE_ref are the oracle's unrounded
float64 results on the exact (widened) inputs the device sees.
"""
import math

import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd.inputs import (WORKLOADS, head_row_samples, random_qkv, sample_rows,
                                                   workload_inputs)
from oracle import ref
from tests.parity import TOL, check_case, compare, run_gpu, say, widen

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ worked row (pages)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_worked_row_through_kernel(dtype):
    """The pages' worked row (1,3 | 2,5): q = e0, K[:,0] = (1,3,2,5), V[:, :4] = I, scale 1.

    Exact in bf16 and fp32; exercises the key-tail mask (4 valid keys of a 64-key tile).
    """
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    d = 64
    q = torch.zeros(1, 1, 1, d, dtype=tdt); q[0, 0, 0, 0] = 1
    k = torch.zeros(1, 1, 4, d, dtype=tdt); k[0, 0, :, 0] = torch.tensor([1, 3, 2, 5], dtype=tdt)
    v = torch.zeros(1, 1, 4, d, dtype=tdt); v[0, 0, :, :4] = torch.eye(4, dtype=tdt)
    o, lse = run_gpu(q, k, v, False, 1.0)
    x = np.array([1.0, 3.0, 2.0, 5.0])
    p = np.exp(x - 5) / np.exp(x - 5).sum()
    tol = TOL[dtype]
    assert np.max(np.abs(o[0, 0, 0, :4] - p)) <= tol["o"]
    assert np.all(o[0, 0, 0, 4:] == 0)
    assert abs(lse[0, 0, 0] - (5 + math.log(1.2034379904932109))) <= tol["lse"]
    assert abs(lse[0, 0, 0] - (5 + math.log(1.203))) <= 1e-3   # the page's printed l


# --------------------------------------------- small and ragged shapes, full check
SHAPES = [
    # B, H, Lq,  Lk,  d
    (1, 1, 1, 1, 64),
    (1, 2, 2, 2, 128),
    (1, 1, 1, 300, 64),
    (1, 1, 300, 1, 128),
    (2, 3, 129, 129, 64),
    (1, 2, 257, 255, 128),
    (1, 1, 64, 64, 128),
    (1, 1, 65, 63, 64),
    (2, 1, 127, 1000, 128),
    (1, 2, 1000, 77, 128),
    (1, 1, 384, 384, 64),
    (1, 1, 500, 500, 128),
    (1, 2, 129, 129, 32),
    (2, 1, 300, 257, 32),
    (1, 1, 1, 1, 32),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_parity_ragged(shape, causal, dtype):
    B, H, Lq, Lk, d = shape
    q, k, v = random_qkv(B, H, Lq, Lk, d, dtype, seed=sum(shape) + 7 * causal)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))
    check_case("ragged %s %s" % (shape, dtype), q, k, v, causal, scale, dtype)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 200, 300, 256), (2, 1, 129, 129, 256), (1, 1, 1, 70, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_parity_head_dim_256(shape, causal):
    """d = 256 (bf16 only: the one-wavefront-per-SIMD instance)."""
    B, H, Lq, Lk, d = shape
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=sum(shape) + 5 * causal)
    check_case("d256 %s" % (shape,), q, k, v, causal, float(np.float32(1 / np.sqrt(d))), "bf16")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 200, 300, 96), (2, 1, 129, 129, 96), (1, 1, 1, 70, 96),
                                   (1, 2, 333, 1000, 96)],
                         ids=lambda s: "x".join(map(str, s)))
def test_parity_head_dim_96(shape, causal):
    """d = 96 (bf16: 192-byte rows staged as 256-byte LDS rows, upper chunks unused)."""
    B, H, Lq, Lk, d = shape
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=sum(shape) + 3 * causal)
    check_case("d96 %s" % (shape,), q, k, v, causal, float(np.float32(1 / np.sqrt(d))), "bf16")


def test_parity_head_dim_96_long_sampled():
    """d = 96 at N=4096 (B=2, H=16, causal), 256 sampled rows of every head."""
    q, k, v = random_qkv(2, 16, 4096, 4096, 96, "bf16", seed=961)
    rows = sample_rows(4096, 256, 962)
    check_case("d96 long", q, k, v, True, float(np.float32(1 / np.sqrt(96))), "bf16", rows=rows)


def test_pages_selfcheck_recipe_through_kernel():
    """The pages' NumPy self-check recipe (rng(0) normal, 100 x 32 for Q, K, V): the
    same draws, rounded to bf16 (and kept fp32), through the kernels."""
    Q, K, V = np.random.default_rng(0).normal(size=(3, 100, 32))
    for dtype, tdt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
        q, k, v = (torch.from_numpy(x[None, None].astype(np.float32)).to(tdt) for x in (Q, K, V))
        check_case("pages' self-check recipe", q, k, v, False, float(np.float32(1 / np.sqrt(32))), dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_parity_large_score_range(causal):
    """Q x 4 (as the ragged workload): peaky rows and frequent max rescaling."""
    q, k, v = random_qkv(2, 2, 700, 900, 128, "bf16", seed=99, q_mult=4.0)
    check_case("peaky", q, k, v, causal, float(np.float32(1 / np.sqrt(128))), "bf16")


# ------------------------------------------------------------ the five workloads
def _rows_for(name, w):
    """Every row of every head, except the N=16384 workload: 2048 seeded rows per
    head, each against its full causal prefix."""
    if name == "B1_H16_L16384_d128_bf16_causal":
        return head_row_samples(w, 2048)
    return None


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_parity_workload(name):
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    check_case(name, q, k, v, w.causal, w.scale, w.dtype, rows=_rows_for(name, w))


# ----------------------------------------------------------- closed forms, edges
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_closed_forms(dtype):
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    B, H, L, d = 1, 2, 200, 128
    _, _, v = random_qkv(B, H, L, L, d, dtype, seed=3)
    q, _, _ = random_qkv(B, H, L, L, d, dtype, seed=4)
    zeros = torch.zeros(B, H, L, d, dtype=tdt)
    for causal in (False, True):
        o, lse = run_gpu(q, zeros, v, causal, 0.125)
        vv = widen(v)
        n = np.arange(1, L + 1) if causal else np.full(L, L)
        mean = np.cumsum(vv, axis=2) / n[None, None, :, None] if causal else np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
        assert np.max(np.abs(o - mean)) <= TOL[dtype]["o"]
        assert np.max(np.abs(lse - np.log(n)[None, None])) <= TOL[dtype]["lse"]
    const = torch.full((B, H, L, d), -1.75, dtype=tdt)
    k = random_qkv(B, H, L, L, d, dtype, seed=5)[1]
    o, _ = run_gpu(q, k, const, False, 0.125)
    assert np.max(np.abs(o + 1.75)) <= TOL[dtype]["o"]
    o, lse = run_gpu(q, k, v, True, 0.125)       # causal row 0 sees key 0 only
    assert np.max(np.abs(o[:, :, 0] - widen(v)[:, :, 0])) <= TOL[dtype]["o"]
    want = 0.125 * np.einsum("bhd,bhd->bh", widen(q)[:, :, 0], widen(k)[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - want)) <= TOL[dtype]["lse"]


def test_bitwise_repeatable():
    q, k, v = (t.cuda() for t in random_qkv(1, 4, 1500, 1500, 128, "bf16", seed=8))
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_error_paths_on_device():
    q = torch.zeros(1, 1, 8, 80, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FA2Error) as e:
        fa.forward(q, q, q)
    assert e.value.status == 3
    buf = torch.zeros(1 + 1 * 1 * 8 * 64, dtype=torch.bfloat16, device="cuda")
    mis = buf[1:].view(1, 1, 8, 64)               # 2-byte offset: misaligned
    good = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FA2Error) as e:
        fa.forward(mis, good, good)
    assert e.value.status == 5


def test_output_rows_all_written():
    """Ragged Lq: every row of o and lse is overwritten (buffers start as NaN)."""
    q, k, v = (t.cuda() for t in random_qkv(1, 3, 333, 129, 64, "bf16", seed=9))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 3, 333), float("nan"), device="cuda")
    fa.forward(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_wrapper_rejects_mismatched_outputs():
    """The library trusts shapes; the Python wrapper refuses outputs it would overrun."""
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 2, 64, device="cuda")
    bad_outs = [torch.zeros(1, 2, 32, 64, dtype=torch.bfloat16, device="cuda"),        # too small
                torch.zeros(1, 2, 64, 64, dtype=torch.float16, device="cuda"),         # wrong dtype
                torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16, device="cuda")[..., ::2]]   # strided
    for out in bad_outs:
        with pytest.raises(ValueError):
            fa.forward(q, q, q, out=out, lse=lse)
    with pytest.raises(ValueError):
        fa.forward(q, q, q, lse=torch.zeros(1, 2, 32, device="cuda"))
    o, l = fa.forward(q, q, q)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, o, l, q, dq=torch.zeros(1, 2, 64, 32, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.merge_partials(torch.zeros(2, 3, 64, device="cuda"), torch.zeros(2, 3, device="cuda"),
                          out=torch.zeros(2, 64, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["one-pass", "split-decode", "split-mfma"])
def test_max_keys_per_head(path):
    """Lk at the one-head limit ((Lk + 64) d 2 bytes < 2^31 at d = 128: 32-bit tile
    offsets up to 2 GiB).  K = 0 except five hot keys (first, early, middle, in the
    last full tile, last) whose first component is 1; V = 1 except distinct hot rows.
    With scale 1, a query 30 e_0 scores 30 on the hot keys and 0 elsewhere, so
    O = ((Lk - h) + e^30 sum V_hot) / Z and LSE = ln Z, Z = (Lk - h) + h e^30, in closed
    form; query 0 gives the plain mean over all Lk keys; query -30 e_0 almost only
    the ones."""
    d, Lk = 128, (1 << 23) - 65
    Lq = 5 if path == "split-mfma" else 3
    say("case max keys per head: Lk=%d d=%d path=%s" % (Lk, d, path))
    hot = np.array([0, 1000, Lk // 2 + 17, Lk - 70, Lk - 1])
    h = len(hot)
    q = torch.zeros(1, 1, Lq, d, dtype=torch.bfloat16, device="cuda")
    q[0, 0, 0, 0] = 30.0
    q[0, 0, 2, 0] = -30.0
    if Lq > 3:
        q[0, 0, 3:, 0] = 30.0
    k = torch.zeros(1, 1, Lk, d, dtype=torch.bfloat16, device="cuda")
    k[0, 0, torch.from_numpy(hot).cuda(), 0] = 1.0
    v = torch.ones(1, 1, Lk, d, dtype=torch.bfloat16, device="cuda")
    vh = (torch.arange(h, dtype=torch.float32)[:, None] * 0.5 + 2.0 +
          torch.arange(d, dtype=torch.float32)[None, :] / 64.0).to(torch.bfloat16)
    v[0, 0, torch.from_numpy(hot).cuda()] = vh.cuda()
    splits = None if path == "one-pass" else 0
    o, lse = fa.forward(q, k, v, scale=1.0, num_splits=splits)
    torch.cuda.synchronize()
    o, lse = o[0, 0].double().cpu().numpy(), lse[0, 0].double().cpu().numpy()
    del k, v
    vsum = vh.double().numpy().sum(axis=0)
    n = Lk - h
    want_o, want_l = [], []
    for s in [30.0, 0.0, -30.0] + [30.0] * (Lq - 3):
        z = n + h * np.exp(s)
        want_o.append((n + np.exp(s) * vsum) / z)
        want_l.append(np.log(z))
    eo = float(np.max(np.abs(o - np.array(want_o))))
    el = float(np.max(np.abs(lse - np.array(want_l))))
    say("  max|dO|=%.3e  max|dLSE|=%.3e" % (eo, el))
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]
