"""Pins for the CPU oracle (no GPU).

The oracle is pinned here to things other than itself: the worked row the pages
print, library routines (scipy's softmax / logsumexp with numpy matmul, PyTorch's
float64 CPU attention), closed forms, invariants, and brute force with exact
summation on tiny inputs.  ``test_planted_mistakes_are_caught`` plants plausible
mistakes in copies of the oracle's C source and checks that the pins catch each.
"""
import ctypes
import json
import math
import os
import subprocess

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attn_ref.c")


# --------------------------------------------------------------------------- pages
def test_worked_row_online_trace_matches_page():
    """The worked row (1,3 | 2,5): m=3, l=1.135 after block 1; m=5, l=1.203 after block 2."""
    g = json.load(open(os.path.join(GOLDEN, "worked_row_online_softmax.json")))
    _, trace = ref.online_softmax(g["row"], block=g["block"])
    tol = 0.5 * 10 ** (-g["printed_decimals"])
    assert len(trace) == len(g["printed_after_block"])
    for (m, l), want in zip(trace, g["printed_after_block"]):
        assert m == want["m"]
        assert abs(l - want["l"]) <= tol
    # the closed forms the page writes next to the numbers
    assert trace[0][1] == pytest.approx(math.exp(-2) + 1, abs=1e-15)
    assert trace[1][1] == pytest.approx((math.exp(-2) + 1) * math.exp(-2) + math.exp(-3) + 1, abs=1e-15)


def test_worked_row_online_equals_three_pass():
    """The page states the two-block result equals computing the row at once."""
    x = [1.0, 3.0, 2.0, 5.0]
    p_online, trace = ref.online_softmax(x, block=2)
    p3 = ref.softmax_3pass(x)
    np.testing.assert_allclose(p_online, p3, rtol=1e-15, atol=0)
    m_all = max(x)
    l_all = sum(math.exp(v - m_all) for v in x)
    assert trace[-1][0] == m_all and trace[-1][1] == pytest.approx(l_all, rel=1e-15)


def test_oracle_on_worked_row():
    """The worked row through the attention oracle: q = e0, K[:,0] = (1,3,2,5), V = I."""
    d = 4
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, 4, d)); k[0, 0, :, 0] = [1, 3, 2, 5]
    v = np.eye(4).reshape(1, 1, 4, 4)
    o, lse = ref.attention_f64(q, k, v, 1.0, False)
    x = np.array([1.0, 3.0, 2.0, 5.0])
    l = np.exp(x - 5).sum()
    np.testing.assert_allclose(o[0, 0, 0], np.exp(x - 5) / l, rtol=1e-14)
    assert lse[0, 0, 0] == pytest.approx(5 + math.log(l), abs=1e-14)
    assert lse[0, 0, 0] == pytest.approx(5 + math.log(1.203), abs=1e-3)  # page's printed l


# ------------------------------------------------------------------ pin helpers
def _scipy_attention(q, k, v, scale, causal):
    """Library-routine route: numpy matmul for S, scipy softmax / logsumexp."""
    S = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        Lq, Lk = S.shape[-2:]
        vis = np.arange(Lk)[None, :] <= np.arange(Lq)[:, None]
        S = np.where(vis, S, -np.inf)
    return softmax(S, axis=-1) @ v, logsumexp(S, axis=-1)


def _torch_sdpa_f64(q, k, v, scale, causal):
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=bool(causal), scale=float(scale))
    return o.numpy()


def _brute_force(q, k, v, scale, causal):
    """Exact-sum brute force, no max shift: w_j = e^{s_j} / sum e^{s}, for tiny, tame inputs."""
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    o = np.zeros((B, H, Lq, d)); lse = np.zeros((B, H, Lq))
    for b in range(B):
        for h in range(H):
            for i in range(Lq):
                vis = range(min(i + 1, Lk)) if causal else range(Lk)
                e = [math.exp(scale * math.fsum(q[b, h, i, t] * k[b, h, j, t] for t in range(d))) for j in vis]
                z = math.fsum(e)
                for t in range(d):
                    o[b, h, i, t] = math.fsum(e[n] * v[b, h, j, t] for n, j in enumerate(vis)) / z
                lse[b, h, i] = math.log(z)
    return o, lse


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


# Each pin takes an attention callable attn(q,k,v,scale,causal[,rows]) -> (o, lse)
# and raises AssertionError when the callable is wrong.
def pin_scipy(attn):
    rng = np.random.default_rng(11)
    for (B, H, Lq, Lk, d, causal) in [(1, 2, 5, 9, 8, False), (2, 1, 9, 9, 16, True),
                                      (1, 1, 13, 6, 4, True), (1, 1, 6, 13, 3, True),
                                      (1, 1, 17, 31, 64, False)]:
        q, k, v = _rand((B, H, Lq, d), rng), _rand((B, H, Lk, d), rng), _rand((B, H, Lk, d), rng)
        scale = 1 / math.sqrt(d)
        o, lse = attn(q, k, v, scale, causal)
        o_ref, lse_ref = _scipy_attention(q, k, v, scale, causal)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def pin_torch_sdpa(attn):
    rng = np.random.default_rng(12)
    for (Lq, Lk, d, causal) in [(33, 33, 32, True), (20, 47, 64, False), (47, 20, 16, True), (7, 19, 5, True)]:
        q, k, v = _rand((2, 3, Lq, d), rng), _rand((2, 3, Lk, d), rng), _rand((2, 3, Lk, d), rng)
        scale = 0.37
        o, _ = attn(q, k, v, scale, causal)
        np.testing.assert_allclose(o, _torch_sdpa_f64(q, k, v, scale, causal), rtol=0, atol=1e-12)


def pin_brute_force(attn):
    rng = np.random.default_rng(13)
    for Lq in (1, 2, 5, 9):
        for Lk in (1, 3, 8):
            for d in (1, 2, 64):
                for causal in (False, True):
                    q = _rand((1, 2, Lq, d), rng, 0.5)
                    k = _rand((1, 2, Lk, d), rng, 0.5)
                    v = _rand((1, 2, Lk, d), rng)
                    scale = 1 / math.sqrt(d)
                    o, lse = attn(q, k, v, scale, causal)
                    ob, lb = _brute_force(q, k, v, scale, causal)
                    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
                    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


def pin_closed_forms(attn):
    rng = np.random.default_rng(14)
    Lq, Lk, d = 12, 12, 8
    q, v = _rand((1, 1, Lq, d), rng), _rand((1, 1, Lk, d), rng)
    # K = 0: uniform weights over the visible keys
    for causal in (False, True):
        o, lse = attn(q, np.zeros((1, 1, Lk, d)), v, 0.3, causal)
        for i in range(Lq):
            n = min(i + 1, Lk) if causal else Lk
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), atol=1e-13)
            assert lse[0, 0, i] == pytest.approx(math.log(n), abs=1e-13)
    # Lk = 1: O = V0, LSE = scale q.k0
    k1 = _rand((1, 1, 1, d), rng)
    o, lse = attn(q, k1, v[:, :, :1], 0.3, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 0], (Lq, d)), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], 0.3 * q[0, 0] @ k1[0, 0, 0], atol=1e-13)
    # V = c: O = c
    k = _rand((1, 1, Lk, d), rng)
    o, _ = attn(q, k, np.full((1, 1, Lk, d), -1.75), 0.3, False)
    np.testing.assert_allclose(o, -1.75, atol=1e-14)
    # causal row 0 sees only key 0
    o, lse = attn(q, k, v, 0.3, True)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-14)
    assert lse[0, 0, 0] == pytest.approx(0.3 * q[0, 0, 0] @ k[0, 0, 0], abs=1e-13)


def pin_invariants(attn):
    rng = np.random.default_rng(15)
    Lq, Lk, d = 10, 7, 8
    q, k, v = _rand((1, 2, Lq, d), rng), _rand((1, 2, Lk, d), rng), _rand((1, 2, Lk, d), rng)
    scale = 0.45
    for causal in (False, True):
        o, lse = attn(q, k, v, scale, causal)
        # shift every key by the same vector u: O unchanged, LSE moves by scale*q.u
        u = _rand((d,), rng)
        o2, lse2 = attn(q, k + u, v, scale, causal)
        np.testing.assert_allclose(o2, o, atol=1e-12)
        np.testing.assert_allclose(lse2, lse + scale * (q @ u), atol=1e-12)
        # LSE bounds: m <= LSE <= m + ln(#visible)
        S = scale * np.einsum("bhid,bhjd->bhij", q, k)
        for i in range(Lq):
            n = min(i + 1, Lk) if causal else Lk
            m = S[..., i, :n].max(axis=-1)
            assert np.all(lse[..., i] >= m - 1e-12) and np.all(lse[..., i] <= m + math.log(n) + 1e-12)
    # joint permutation of keys and values (non-causal): no change
    perm = rng.permutation(Lk)
    o, lse = attn(q, k, v, scale, False)
    o3, lse3 = attn(q, k[:, :, perm], v[:, :, perm], scale, False)
    np.testing.assert_allclose(o3, o, atol=1e-13)
    np.testing.assert_allclose(lse3, lse, atol=1e-13)
    # V = I (Lk <= d): rows of O are the softmax weights: non-negative, sum to 1
    vI = np.broadcast_to(np.eye(Lk, d), (1, 2, Lk, d)).copy()
    oI, lseI = attn(q, k, vI, scale, False)
    assert np.all(oI >= 0)
    np.testing.assert_allclose(oI.sum(axis=-1), 1.0, atol=1e-13)
    np.testing.assert_allclose(oI[..., :Lk], np.exp(S - lseI[..., None]), atol=1e-13)


def pin_sampled_rows(attn):
    rng = np.random.default_rng(16)
    Lq, Lk, d = 40, 40, 8
    q, k, v = _rand((2, 2, Lq, d), rng), _rand((2, 2, Lk, d), rng), _rand((2, 2, Lk, d), rng)
    rows = np.stack([np.sort(rng.choice(Lq, 9, replace=False)) for _ in range(4)])
    for causal in (False, True):
        o, lse = attn(q, k, v, 0.4, causal)
        os_, lses = attn(q, k, v, 0.4, causal, rows=rows)
        for bh in range(4):
            b, h = divmod(bh, 2)
            np.testing.assert_allclose(os_[b, h], o[b, h, rows[bh]], atol=0)
            np.testing.assert_allclose(lses[b, h], lse[b, h, rows[bh]], atol=0)


PINS = [pin_scipy, pin_torch_sdpa, pin_brute_force, pin_closed_forms, pin_invariants, pin_sampled_rows]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ref.attention_f64)


# ----------------------------------------------------- the tiled method on CPU
def test_p3_selfcheck_shape_tiled_equals_definition():
    """The pages' self-check recipe: rng(0) normal (3,100,32), K/V blocks of 16, ragged."""
    Q, K, V = np.random.default_rng(0).normal(size=(3, 100, 32))
    o_def, lse_def = ref.attention_f64(Q[None, None], K[None, None], V[None, None], 1 / np.sqrt(32), False)
    for Br in (100, 7):
        o, lse = ref.flash_attention2_tiled(Q, K, V, 1 / np.sqrt(32), False, Br=Br, Bc=16)
        np.testing.assert_allclose(o, o_def[0, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_def[0, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_three_pass_online_tiled_agree(causal):
    rng = np.random.default_rng(21)
    x = rng.standard_normal(97) * 6
    p3 = ref.softmax_3pass(x)
    for blk in (1, 2, 3, 16, 64, 97):
        p, _ = ref.online_softmax(x, block=blk)
        np.testing.assert_allclose(p, p3, rtol=1e-14, atol=0)
    Lq, Lk, d = 70, 70 if causal else 83, 16
    q, k, v = rng.standard_normal((Lq, d)), rng.standard_normal((Lk, d)), rng.standard_normal((Lk, d))
    o_def, lse_def = ref.attention_f64(q[None, None], k[None, None], v[None, None], 0.3, causal)
    for Br, Bc in [(1, 1), (2, 3), (16, 16), (64, 64), (Lq, Lk), (5, 64)]:
        o, lse = ref.flash_attention2_tiled(q, k, v, 0.3, causal, Br, Bc)
        np.testing.assert_allclose(o, o_def[0, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse_def[0, 0], rtol=0, atol=1e-13)


def test_oracle_rejects_bad_arguments():
    q = np.zeros((1, 1, 4, 8)); k = np.zeros((1, 1, 4, 8))
    with pytest.raises(ValueError):
        ref.attention_f64(q, k, k, 1.0, False, rows=np.array([0, 4]))
    with pytest.raises(ValueError):
        ref.attention_f64(q, k, k, 1.0, False, rows=np.array([-1]))


# ----------------------------------------------------- planted mistakes (CPU only)
MUTANTS = {
    "causal_off_by_one": ("nvis = i + 1; /* keys 0..i */", "nvis = i + 2; /* keys 0..i */"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "exp_sign_flipped": ("const double p = exp(s[j] - m) / l;", "const double p = exp(m - s[j]) / l;"),
    "lse_log2": ("*lse = m + log(l);", "*lse = m + log2(l);"),
    "v_read_from_k": ("o[t] += p * V[(size_t)j * d + t];", "o[t] += p * K[(size_t)j * d + t];"),
    "divide_dropped": ("const double p = exp(s[j] - m) / l;", "const double p = exp(s[j] - m);"),
    "k_transposed_index": ("dot += q[t] * K[(size_t)j * d + t];", "dot += q[t] * K[((size_t)t * nvis + j) % ((size_t)nvis * d)];"),
    "row_index_from_sample": ("const double *qi = q + ((size_t)bh * Lq + i) * d;",
                              "const double *qi = q + ((size_t)bh * Lq + r) * d;"),
    "causal_ignored": ("if (causal && i + 1 < Lk)", "if (0 && i + 1 < Lk)"),
}


def _load_mutant(name, tmp_path):
    src = open(ORACLE_SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src.replace(old, new))
    so = tmp_path / ("mut_%s.so" % name)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    lib.oracle_attention_f64.restype = ctypes.c_int
    lib.oracle_attention_f64.argtypes = ref._lib().oracle_attention_f64.argtypes

    def attn(q, k, v, scale, causal, rows=None):
        saved = ref._LIB
        ref._LIB = lib
        try:
            return ref.attention_f64(q, k, v, scale, causal, rows=rows, nthreads=1)
        finally:
            ref._LIB = saved
    return attn


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, tmp_path):
    attn = _load_mutant(name, tmp_path)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name


# --------------------------------------------------------------- merge of partials
# ref.merge_partials is pinned to the definition (attention over all keys, whose
# oracle is pinned above), to scipy's logsumexp, and to closed forms.

MERGE_BOUNDS = [(0, 37), (37, 38), (38, 160), (160, 300)]


def _shard_inputs(seed=21):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((2, 3, 50, 64))
    k = rng.standard_normal((2, 3, 300, 64))
    v = rng.standard_normal((2, 3, 300, 64))
    return q, k, v, 0.2


def _shard_results(q, k, v, scale, bounds):
    """Oracle attention of every query against each key shard [a, b), non-causal."""
    parts = [ref.attention_f64(q, k[:, :, a:b], v[:, :, a:b], scale, False) for a, b in bounds]
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


def merge_pin_definition(merge):
    """Merging the results over key shards gives attention over all keys."""
    q, k, v, scale = _shard_inputs()
    o_parts, l_parts = _shard_results(q, k, v, scale, MERGE_BOUNDS)
    o, lse = merge(o_parts, l_parts)
    o_ref, l_ref = ref.attention_f64(q, k, v, scale, False)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(lse - l_ref)) < 1e-12


def merge_pin_logsumexp(merge):
    """LSE of the merge is scipy's logsumexp over the parts; O is a convex combination."""
    rng = np.random.default_rng(5)
    l_parts = rng.normal(0.0, 6.0, size=(5, 40))
    o_parts = rng.standard_normal((5, 40, 8))
    o, lse = merge(o_parts, l_parts)
    assert np.max(np.abs(lse - logsumexp(l_parts, axis=0))) < 1e-12
    w = softmax(l_parts, axis=0)
    assert np.max(np.abs(o - np.einsum("sr,srd->rd", w, o_parts))) < 1e-12


def merge_pin_closed_forms(merge):
    """Equal halves: L + ln 2 and the mean; weights 3:1 at L = 1000 (no overflow)."""
    o1 = np.array([[1.0, -2.0, 0.5]])
    o2 = np.array([[3.0, 4.0, -0.5]])
    o, lse = merge(np.stack([o1, o2]), np.array([[0.7], [0.7]]))
    assert abs(lse[0] - (0.7 + math.log(2))) < 1e-14
    assert np.max(np.abs(o - (o1 + o2) / 2)) < 1e-14
    o, lse = merge(np.stack([o1, o2]), np.array([[1000.0], [1000.0 - math.log(3)]]))
    assert abs(lse[0] - (1000.0 + math.log(4 / 3))) < 1e-11
    assert np.max(np.abs(o - (0.75 * o1 + 0.25 * o2))) < 1e-13


def merge_pin_empty_parts(merge):
    """A -inf part is ignored (its O is not read); an all-empty row is O = 0, L = -inf."""
    o1 = np.array([[1.0, 2.0], [5.0, 6.0]])
    junk = np.full((2, 2), np.nan)
    o, lse = merge(np.stack([junk, o1, junk]),
                   np.array([[-np.inf, -np.inf], [0.25, -np.inf], [-np.inf, -np.inf]]))
    assert np.array_equal(o[0], o1[0]) and lse[0] == 0.25
    assert np.array_equal(o[1], [0.0, 0.0]) and lse[1] == -np.inf


MERGE_PINS = [merge_pin_definition, merge_pin_logsumexp, merge_pin_closed_forms, merge_pin_empty_parts]


@pytest.mark.parametrize("pin", MERGE_PINS, ids=lambda f: f.__name__)
def test_merge_pin(pin):
    pin(ref.merge_partials)


def test_merge_order_invariant():
    q, k, v, scale = _shard_inputs(seed=3)
    o_parts, l_parts = _shard_results(q, k, v, scale, MERGE_BOUNDS)
    perm = [2, 0, 3, 1]
    o1, l1 = ref.merge_partials(o_parts, l_parts)
    o2, l2 = ref.merge_partials(o_parts[perm], l_parts[perm])
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13


# Plausible mistakes in the merge; each must fail at least one merge pin.
MERGE_MUTANTS = {
    "weight_without_max": ("np.exp(l2 - safe)", "np.exp(l2)"),
    "max_instead_of_logsumexp": ("np.logaddexp(lse, l2)", "np.maximum(lse, l2)"),
    "unweighted_sum": ("w1[..., None] * o + w2[..., None] * o2", "o + o2"),
    "old_weight_from_new_part": ("np.exp(lse - safe)", "np.exp(l2 - safe)"),
    "empty_part_read": ("np.where(np.isneginf(l2)[..., None], 0.0, o_parts[s])", "o_parts[s]"),
}


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_planted_mistakes_are_caught(name):
    import inspect
    import textwrap
    old, new = MERGE_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(ref.merge_partials))
    assert src.count(old) == 1, old
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    caught = []
    for pin in MERGE_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ns["merge_partials"])
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every merge pin" % name
