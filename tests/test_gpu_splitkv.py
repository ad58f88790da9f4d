"""Parity of the split-KV forward (partials + merge, through the C ABI) and of
the stand-alone merge with the float64 oracle.

Bars as for the one-pass bf16 path: max|O - O_ref| <= 2e-2, max|LSE - LSE_ref|
<= 1e-3 against the oracle's unrounded results (attention over all keys for the
split path; the oracle's merge for fa2_merge_partials, whose fp32 logsumexp is
held to 1e-5).
"""
import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd.inputs import (DECODE_WORKLOADS, WORKLOADS, head_row_samples,
                                                   random_qkv, workload_inputs)
from oracle import ref
from tests.parity import check_case, compare, say, widen

pytestmark = pytest.mark.gpu


def _scale(d):
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


SHAPES = [
    # B, H, Lq,  Lk,   d
    (1, 1, 1, 1, 64),          # one key: every split but one is empty
    (1, 1, 1, 300, 64),        # single query
    (2, 3, 129, 129, 64),
    (1, 2, 257, 255, 128),
    (2, 1, 127, 1000, 128),
    (1, 2, 1000, 77, 128),
    (1, 1, 500, 500, 128),
    (1, 2, 300, 5000, 128),
    (1, 2, 200, 700, 32),
    (1, 1, 150, 900, 256),
    (1, 2, 150, 900, 96),
]


@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_splitkv_ragged(shape, causal, splits):
    B, H, Lq, Lk, d = shape
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=sum(shape) + 7 * causal + 100 * splits)
    check_case("split ragged %s S=%d" % (shape, splits), q, k, v, causal, _scale(d), "bf16",
               num_splits=splits)


DECODE_SHAPES = [
    # B, H, Lq, Lk, d   (Lq <= 4: the split-KV path runs the decoding kernel)
    (1, 4, 1, 4097, 128),
    (2, 3, 2, 1000, 64),
    (1, 2, 3, 777, 96),
    (1, 2, 4, 2048, 256),
    (3, 1, 4, 100, 32),
    (1, 1, 1, 5, 128),      # more splits than keys: most ranges empty
    (2, 2, 3, 3, 64),
]


@pytest.mark.parametrize("splits", [2, 7, 0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_kernel_parity(shape, causal, splits):
    B, H, Lq, Lk, d = shape
    q, k, v = random_qkv(B, H, Lq, Lk, d, "bf16", seed=sum(shape) + 3 * causal + splits)
    check_case("decode %s S=%d" % (shape, splits), q, k, v, causal, _scale(d), "bf16", num_splits=splits)


def test_decode_kernel_peaky_scores():
    """Q x 8 (scores spread over tens of units): the per-step max moves often."""
    q, k, v = random_qkv(1, 2, 2, 3000, 128, "bf16", seed=77, q_mult=8.0)
    check_case("decode peaky", q, k, v, False, _scale(128), "bf16", num_splits=0)


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_more_splits_than_tiles(causal):
    """S = 128 on 5 K/V tiles: most ranges are empty, and (causal) most rows of a
    non-empty range see none of its keys."""
    q, k, v = random_qkv(1, 2, 300, 300, 128, "bf16", seed=31 + causal)
    check_case("split S=max", q, k, v, causal, _scale(128), "bf16", num_splits=fa.FA2_MAX_SPLITS)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 300, 5000, 128), (2, 3, 129, 129, 64), (1, 1, 1, 777, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_one_split_is_bitwise_the_one_pass_result(shape, causal):
    B, H, Lq, Lk, d = shape
    q, k, v = (t.cuda() for t in random_qkv(B, H, Lq, Lk, d, "bf16", seed=41))
    o1, l1 = fa.forward(q, k, v, causal=causal)
    o2, l2 = fa.forward(q, k, v, causal=causal, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 300, 64, 128), (2, 3, 129, 50, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_single_nonempty_range_is_bitwise_the_one_pass_result(shape, causal):
    """One K/V tile and 3 splits: two ranges are empty, the third holds the tile
    and does the one-pass arithmetic; the merge weights it by exactly 1."""
    B, H, Lq, Lk, d = shape
    q, k, v = (t.cuda() for t in random_qkv(B, H, Lq, Lk, d, "bf16", seed=43))
    o1, l1 = fa.forward(q, k, v, causal=causal)
    o2, l2 = fa.forward(q, k, v, causal=causal, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_ragged_workload_auto_splits():
    """The Lq=1000 / Lk=7777 workload (192 query tiles) with the library's split count, every row."""
    w = WORKLOADS["B3_H8_Lq1000_Lk7777_d128_bf16_q4"]
    say("auto splits: %d" % fa.fa2_splitkv_num_splits(w.B, w.H, w.Lq, w.Lk, w.d, int(w.causal)))
    q, k, v = workload_inputs(w)
    check_case(w.name + " auto", q, k, v, w.causal, w.scale, w.dtype, num_splits=0)


def test_splitkv_headline_workload_sampled_rows():
    """The causal 2x32x4096 workload split in 3, on 384 seeded rows per head."""
    w = WORKLOADS["B2_H32_L4096_d128_bf16_causal"]
    q, k, v = workload_inputs(w)
    check_case(w.name + " S=3", q, k, v, w.causal, w.scale, w.dtype, rows=head_row_samples(w, 384),
               num_splits=3)


@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_splitkv_decode_workload(name):
    """One query per head against a 128K-key cache, auto split count, every row."""
    w = DECODE_WORKLOADS[name]
    say("auto splits: %d" % fa.fa2_splitkv_num_splits(w.B, w.H, w.Lq, w.Lk, w.d, int(w.causal)))
    q, k, v = workload_inputs(w)
    check_case(name, q, k, v, w.causal, w.scale, w.dtype, num_splits=0)


def test_splitkv_repeatable_and_all_rows_written():
    q, k, v = (t.cuda() for t in random_qkv(1, 3, 333, 2000, 64, "bf16", seed=9))
    outs = []
    for _ in range(2):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((1, 3, 333), float("nan"), device="cuda")
        ws = torch.full((fa.fa2_splitkv_workspace_bytes(1, 3, 333, 2000, 64, 1, 5),), 255,
                        dtype=torch.uint8, device="cuda")      # NaN-filled workspace
        fa.forward(q, k, v, causal=True, out=o, lse=lse, num_splits=5, workspace=ws)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0][0]).all() and torch.isfinite(outs[0][1]).all()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_splitkv_workspace_too_small():
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    need = fa.fa2_splitkv_workspace_bytes(1, 1, 64, 64, 64, 0, 2)
    ws = torch.zeros(need - 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FA2Error) as e:
        fa.forward(q, q, q, num_splits=2, workspace=ws)
    assert e.value.status == 8


# ------------------------------------------------------ stand-alone merge kernel
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_merge_partials_matches_oracle(d):
    """Partials: the oracle's attention over key shards (rounded to fp32), plus one
    part that is empty (-inf, NaN output) for every row and one empty for some rows."""
    B, H, Lq, Lk = 2, 3, 77, 900
    q, k, v = (widen(t) for t in random_qkv(B, H, Lq, Lk, d, "bf16", seed=51))
    bounds = [(0, 100), (100, 101), (101, 600), (600, 900)]
    parts = [ref.attention_f64(q, k[:, :, a:b], v[:, :, a:b], 0.11, False) for a, b in bounds]
    o_parts = np.stack([p[0] for p in parts] + [np.full((B, H, Lq, d), np.nan)]).astype(np.float32)
    l_parts = np.stack([p[1] for p in parts] + [np.full((B, H, Lq), -np.inf)]).astype(np.float32)
    l_parts[1, :, :, ::3] = -np.inf                  # part 1 empty on every third row
    o_parts[1, :, :, ::3] = np.nan
    o_ref, l_ref = ref.merge_partials(o_parts, l_parts)
    o, lse = fa.merge_partials(torch.from_numpy(o_parts).cuda(), torch.from_numpy(l_parts).cuda())
    torch.cuda.synchronize()
    eo = float(np.max(np.abs(o.double().cpu().numpy() - o_ref)))
    el = float(np.max(np.abs(lse.double().cpu().numpy() - l_ref)))
    say("  merge d=%d  max|dO|=%.3e  max|dLSE|=%.3e" % (d, eo, el))
    assert eo <= 2e-2 and el <= 1e-5


def test_merge_all_empty_row():
    o_parts = torch.full((3, 4, 64), float("nan"), device="cuda")
    l_parts = torch.full((3, 4), float("-inf"), device="cuda")
    l_parts[1, 2] = 0.5
    o_parts[1, 2] = 0.25
    o, lse = fa.merge_partials(o_parts, l_parts)
    torch.cuda.synchronize()
    o, lse = o.float().cpu(), lse.cpu()
    assert torch.all(o[[0, 1, 3]] == 0) and torch.all(torch.isneginf(lse[[0, 1, 3]]))
    assert torch.all(o[2] == 0.25) and lse[2] == 0.5
