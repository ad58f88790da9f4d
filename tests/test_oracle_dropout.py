"""Pins for the dropout oracle (no GPU).

The generator is pinned to the known-answer vectors published with Philox4x32-10
(Salmon, Moraes, Dror, Shaw, SC'11; the Random123 library's tests) and to a
second, vectorised implementation of the same definition; the mask to its
keep rate and to the absence of correlation between neighbouring elements; the
attention with dropout to PyTorch's float64 CPU attention arithmetic and autograd
with the same mask, and to the plain oracle when nothing is dropped (t = 256).
``test_planted_mistakes_are_caught`` plants mistakes in copies of the C source.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import torch

from oracle import ref

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attn_dropout_ref.c")

# (counter, key) -> output, Philox4x32-10 known answers
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff,) * 4, (0xffffffff, 0xffffffff), (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


def _philox_np(ctr, key):
    """Philox4x32-10 for arrays of counters [n, 4] and one key: a second implementation."""
    c = [ctr[:, i].astype(np.uint64) for i in range(4)]
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    m32 = np.uint64(0xFFFFFFFF)
    for _ in range(10):
        p0 = np.uint64(0xD2511F53) * c[0]
        p1 = np.uint64(0xCD9E8D57) * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & m32, p1 & m32, ((p0 >> np.uint64(32)) ^ c[3] ^ k1) & m32, p0 & m32]
        k0 = (k0 + np.uint64(0x9E3779B9)) & m32
        k1 = (k1 + np.uint64(0xBB67AE85)) & m32
    return np.stack(c, axis=1).astype(np.uint32)


def _mask_np(B, H, Lq, Lk, seed, offset, t):
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    out = np.empty((B, H, Lq, Lk), dtype=bool)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    for bh in range(B * H):
        ctr = np.stack(np.broadcast_arrays(j // 4, i // 4, np.full_like(i, bh), np.full_like(i, offset)), axis=-1)
        w = _philox_np(ctr.reshape(-1, 4).astype(np.uint32), key).reshape(Lq, Lk, 4)
        word = np.take_along_axis(w, np.broadcast_to((i % 4)[..., None], (Lq, Lk, 1)), axis=2)[..., 0]
        byte = (word >> (8 * (j % 4)).astype(np.uint32)) & 0xFF
        out[bh // H, bh % H] = byte < t
    return out


def _torch_dropout_attention(q, k, v, dout, scale, causal, mask, t):
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2)
    if causal:
        Lq, Lk = s.shape[-2:]
        vis = torch.arange(Lk)[None, :] <= torch.arange(Lq)[:, None]
        s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, dim=-1)
    a = p * torch.from_numpy(mask).double() * (256.0 / t)
    o = a @ tv
    lse = torch.logsumexp(s, dim=-1)
    o.backward(torch.tensor(dout))
    return o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


# ------------------------------------------------------------------ generator
def test_philox_known_answers():
    for ctr, key, want in KAT:
        assert tuple(int(x) for x in ref.philox4x32_10(ctr, key)) == want


def test_philox_second_implementation():
    rng = np.random.default_rng(7)
    ctr = rng.integers(0, 2 ** 32, size=(200, 4), dtype=np.uint64).astype(np.uint32)
    for key in [(0, 0), (0x12345678, 0x9abcdef0)]:
        got = np.stack([ref.philox4x32_10(c, key) for c in ctr])
        np.testing.assert_array_equal(got, _philox_np(ctr, key))
    for ctr_, key_, want in KAT:
        assert tuple(int(x) for x in _philox_np(np.array([ctr_], dtype=np.uint32), key_)[0]) == want


def test_mask_matches_second_implementation_and_rate():
    m = ref.dropout_mask(2, 3, 37, 53, 0x0123456789ABCDEF, 5, 179)
    np.testing.assert_array_equal(m, _mask_np(2, 3, 37, 53, 0x0123456789ABCDEF, 5, 179))
    big = ref.dropout_mask(1, 4, 256, 256, 99, 0, 179)
    n = big.size
    rate, want = big.mean(), 179 / 256
    assert abs(rate - want) <= 5 * math.sqrt(want * (1 - want) / n)
    # neighbours are not correlated (same word, same counter, other counter)
    x = big.astype(np.float64) - want
    for a, b in ((x[..., :-1], x[..., 1:]), (x[..., :-1, :], x[..., 1:, :]), (x[..., :-4], x[..., 4:])):
        corr = (a * b).mean() / (want * (1 - want))
        assert abs(corr) < 0.01
    # a different offset or seed gives a different mask
    assert (ref.dropout_mask(1, 4, 256, 256, 99, 1, 179) != big).mean() > 0.3
    assert (ref.dropout_mask(1, 4, 256, 256, 100, 0, 179) != big).mean() > 0.3


def test_threshold_reading():
    assert ref.dropout_threshold(0.0) == 256 and ref.dropout_threshold(0.1) == 230
    assert ref.dropout_threshold(0.5) == 128 and ref.dropout_threshold(0.999) == 1
    with pytest.raises(ValueError):
        ref.dropout_threshold(1.0)


# ------------------------------------------------------------------ attention
def pin_torch(drop):
    rng = np.random.default_rng(51)
    for (B, H, Lq, Lk, d, causal, t) in [(1, 2, 17, 17, 8, True, 179), (2, 1, 9, 23, 4, False, 128),
                                         (1, 1, 21, 8, 16, True, 230), (1, 1, 5, 5, 3, False, 1)]:
        q, k, v = (rng.standard_normal((B, H, L, d)) for L in (Lq, Lk, Lk))
        dout = rng.standard_normal((B, H, Lq, d))
        seed, offset = 0x1234ABCD5678EF01, 3
        mask = ref.dropout_mask(B, H, Lq, Lk, seed, offset, t)
        got = drop(q, k, v, 0.4, causal, seed, offset, t, dout)
        want = _torch_dropout_attention(q, k, v, dout, 0.4, causal, mask, t)
        for g, w in zip(got, want):
            np.testing.assert_allclose(g, w, rtol=0, atol=1e-12)


def pin_no_drop(drop):
    """t = 256 keeps everything: the plain oracle's output and gradients."""
    rng = np.random.default_rng(52)
    q, k, v = (rng.standard_normal((1, 2, L, 8)) for L in (19, 25, 25))
    dout = rng.standard_normal((1, 2, 19, 8))
    for causal in (False, True):
        o, lse, dq, dk, dv = drop(q, k, v, 0.3, causal, 5, 0, 256, dout)
        o2, lse2 = ref.attention_f64(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, o2, atol=1e-13)
        np.testing.assert_allclose(lse, lse2, atol=1e-13)
        for g, w in zip((dq, dk, dv), ref.attention_bwd_f64(q, k, v, dout, 0.3, causal)):
            np.testing.assert_allclose(g, w, atol=1e-12)


def pin_identities(drop):
    """O is linear in V: <dV, V> = <dO, O>; keys shifted together leave O: sum_j dK_j = 0."""
    rng = np.random.default_rng(53)
    q, k, v = (rng.standard_normal((1, 2, L, 6)) for L in (14, 11, 11))
    dout = rng.standard_normal((1, 2, 14, 6))
    o, _, dq, dk, dv = drop(q, k, v, 0.5, False, 77, 9, 150, dout)
    np.testing.assert_allclose((dv * v).sum(axis=(2, 3)), (dout * o).sum(axis=(2, 3)), atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)


PINS = [pin_torch, pin_no_drop, pin_identities]


def _oracle(q, k, v, scale, causal, seed, offset, t, dout):
    return ref.attention_dropout_f64(q, k, v, scale, causal, seed, offset, t, dout=dout)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_dropout_oracle_pin(pin):
    pin(_oracle)


MUTANTS = {
    "word_byte_swapped": ("return (w[i % 4] >> (8 * (j % 4))) & 0xFFu;", "return (w[j % 4] >> (8 * (i % 4))) & 0xFFu;"),
    "counter_rows_first": ("const uint32_t ctr[4] = {(uint32_t)(j / 4), (uint32_t)(i / 4), (uint32_t)bh, offset};",
                           "const uint32_t ctr[4] = {(uint32_t)(i / 4), (uint32_t)(j / 4), (uint32_t)bh, offset};"),
    "nine_rounds": ("for (int r = 0; r < 10; ++r) {", "for (int r = 0; r < 9; ++r) {"),
    "scale_not_applied": ("const double keep_scale = 256.0 / t;", "const double keep_scale = 1.0;"),
    "row_term_without_dropout": ("                Di += a * da;", "                Di += P[j] * da;"),
    "dp_not_masked": ("const double dp = dropout_byte(bh, i, j, seed, offset) < (uint32_t)t ? da * keep_scale : 0.0;",
                      "const double dp = da * keep_scale;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src.replace(old, new))
    so = tmp_path / ("mut_%s.so" % name)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    real = ref._lib()

    class _Shim:
        oracle_attention_f64 = real.oracle_attention_f64
        oracle_attention_bwd_f64 = real.oracle_attention_bwd_f64
        oracle_attention_bwd_window_f64 = real.oracle_attention_bwd_window_f64
    for fname in ("oracle_philox4x32_10", "oracle_dropout_mask", "oracle_attention_dropout_f64"):
        fn = getattr(lib, fname)
        fn.restype = getattr(real, fname).restype
        fn.argtypes = getattr(real, fname).argtypes
        setattr(_Shim, fname, fn)

    saved = ref._LIB
    ref._LIB = _Shim
    caught = []
    try:
        for check in [test_philox_known_answers, test_mask_matches_second_implementation_and_rate] + \
                [lambda p=p: p(_oracle) for p in PINS]:
            try:
                with np.errstate(all="ignore"):
                    check()
            except (AssertionError, ValueError):
                caught.append(check)
    finally:
        ref._LIB = saved
    assert caught, "planted mistake %r passed every pin" % name
