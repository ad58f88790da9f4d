"""Invariants of exact attention, checked on the HIP forward without the oracle.

Softmax is unchanged when every score of a row moves by the same amount, so
moving every key by one vector u leaves O and moves the logsumexp by
scale * q.u; the keys are a set, so permuting K and V rows together (no mask)
changes nothing; with V = I the rows of O are the attention weights,
non-negative and summing to one; and the logsumexp lies between the row's max
score m and m + ln(#visible keys).  Inputs sit on a grid of 1/8 so that K + u is
exact in bf16 and fp16; bars are the forward's (O 2e-2, LSE 1e-3)."""
import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from tests.parity import say

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


def grid_inputs(B, H, Lq, Lk, d, dtype, seed):
    """Q, K, V with entries n / 8, |n| <= 24 (exact in both 16-bit formats)."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.integers(-24, 25, size=s).astype(np.float32) / 8.0
               for s in ((B, H, Lq, d), (B, H, Lk, d), (B, H, Lk, d)))
    t = DTYPES[dtype]
    return (torch.from_numpy(q).to(t), torch.from_numpy(k).to(t), torch.from_numpy(v).to(t))


def fwd(q, k, v, causal, scale):
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_key_shift(dtype, causal):
    B, H, Lq, Lk, d = 1, 3, 333, 517, 128
    say("case invariant key shift %s causal=%d" % (dtype, causal))
    q, k, v = grid_inputs(B, H, Lq, Lk, d, dtype, seed=81 + causal)
    q = q / 4                                       # keep the scores moderate (still exact)
    scale = float(np.float32(1 / np.sqrt(d)))
    u = torch.from_numpy(np.random.default_rng(82).integers(-2, 3, size=(B, H, 1, d)).astype(np.float32))
    k2 = (k.float() + u).to(k.dtype)
    assert torch.equal(k2.float(), k.float() + u)   # the shift is exact
    o1, l1 = fwd(q, k, v, causal, scale)
    o2, l2 = fwd(q, k2, v, causal, scale)
    qu = np.einsum("bhid,bhjd->bhi", q.double().numpy(), u.double().numpy())
    eo = float(np.abs(o2 - o1).max())
    el = float(np.abs(l2 - (l1 + scale * qu)).max())
    say("  max|O' - O|=%.3e  max|LSE' - LSE - scale q.u|=%.3e" % (eo, el))
    assert eo <= 2e-2 and el <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_joint_key_permutation(dtype):
    B, H, Lq, Lk, d = 2, 2, 200, 450, 64
    say("case invariant permutation %s" % dtype)
    q, k, v = grid_inputs(B, H, Lq, Lk, d, dtype, seed=83)
    q = q / 4
    scale = float(np.float32(1 / np.sqrt(d)))
    perm = torch.from_numpy(np.random.default_rng(84).permutation(Lk))
    o1, l1 = fwd(q, k, v, False, scale)
    o2, l2 = fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), False, scale)
    eo, el = float(np.abs(o2 - o1).max()), float(np.abs(l2 - l1).max())
    say("  max|dO|=%.3e  max|dLSE|=%.3e" % (eo, el))
    assert eo <= 2e-2 and el <= 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_give_weights(causal):
    """V = I (Lk = d): row i of O is the weight row; >= 0, sums to 1."""
    B, H, Lq, d = 1, 2, 300, 128
    say("case invariant V = I causal=%d" % causal)
    q, k, _ = grid_inputs(B, H, Lq, d, d, "bf16", seed=85 + causal)
    v = torch.eye(d, dtype=torch.bfloat16).expand(B, H, d, d).contiguous()
    o, _ = fwd(q / 4, k, v, causal, float(np.float32(1 / np.sqrt(d))))
    assert (o >= 0).all()
    es = float(np.abs(o.sum(axis=-1) - 1.0).max())
    say("  min O=%.3e  max|row sum - 1|=%.3e" % (float(o.min()), es))
    assert es <= 2e-2
    if causal:                                      # no weight on keys after the row
        i, j = np.triu_indices(min(Lq, d), k=1)
        assert (o[:, :, i, j] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_lse_bounds(causal):
    B, H, Lq, Lk, d = 2, 2, 257, 391, 64
    say("case invariant LSE bounds causal=%d" % causal)
    q, k, v = grid_inputs(B, H, Lq, Lk, d, "bf16", seed=87 + causal)
    q = q / 4
    scale = float(np.float32(1 / np.sqrt(d)))
    _, lse = fwd(q, k, v, causal, scale)
    s = scale * np.einsum("bhid,bhjd->bhij", q.double().numpy(), k.double().numpy())
    n_vis = np.full((Lq,), float(Lk))
    if causal:
        s = np.where(np.arange(Lk)[None, :] <= np.arange(Lq)[:, None], s, -np.inf)
        n_vis = np.minimum(np.arange(Lq) + 1.0, Lk)
    m = s.max(axis=-1)
    lo, hi = float((m - lse).max()), float((lse - (m + np.log(n_vis))).max())
    say("  max(m - LSE)=%.3e  max(LSE - m - ln n)=%.3e" % (lo, hi))
    assert lo <= 1e-3 and hi <= 1e-3
