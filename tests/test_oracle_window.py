"""Pins for the sliding-window attention oracle (no GPU).

``ref.attention_window_f64`` (exact attention over keys j with
i - wl <= j <= i + wr, either bound optional) is pinned to PyTorch's float64 CPU
attention with an explicit boolean mask, to the full and causal references it
must reduce to, to the causal reference on reversed sequences (the window
(0, -1) looks forward), to closed forms, and to exact-sum brute force on tiny
inputs including rows that see no key.  ``test_planted_mistakes_are_caught``
plants plausible mistakes in copies of the C source and checks the pins catch each.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import torch

from oracle import ref

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attn_window_ref.c")


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _visible(Lq, Lk, wl, wr):
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    m = np.ones((Lq, Lk), dtype=bool)
    if wl >= 0:
        m &= j >= i - wl
    if wr >= 0:
        m &= j <= i + wr
    return m


WINDOWS = [(-1, -1), (-1, 0), (0, 0), (3, 0), (5, 2), (0, 4), (-1, 3), (2, -1), (40, 40)]


# Each pin takes win(q, k, v, scale, wl, wr[, rows]) -> (o, lse) and raises AssertionError if wrong.
def pin_torch_mask(win):
    rng = np.random.default_rng(41)
    for (Lq, Lk, d) in [(17, 17, 8), (20, 33, 16), (31, 12, 4)]:
        q, k, v = _rand((1, 2, Lq, d), rng), _rand((1, 2, Lk, d), rng), _rand((1, 2, Lk, d), rng)
        for (wl, wr) in WINDOWS:
            m = _visible(Lq, Lk, wl, wr)
            rows = np.nonzero(m.any(axis=1))[0]          # torch gives NaN for empty rows
            o, _ = win(q, k, v, 0.37, wl, wr)
            t = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                attn_mask=torch.from_numpy(m), scale=0.37).numpy()
            np.testing.assert_allclose(o[:, :, rows], t[:, :, rows], rtol=0, atol=1e-12)


def pin_reduces_to_full_and_causal(win):
    rng = np.random.default_rng(42)
    q, k, v = _rand((2, 1, 23, 8), rng), _rand((2, 1, 29, 8), rng), _rand((2, 1, 29, 8), rng)
    for wl, wr, causal in [(-1, -1, False), (-1, 0, True), (-1, 40, False), (40, 0, True)]:
        o, lse = win(q, k, v, 0.5, wl, wr)
        o2, lse2 = ref.attention_f64(q, k, v, 0.5, causal)
        np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)


def pin_reversed_causal(win):
    """Window (0, -1) sees keys j >= i: the causal mask on the reversed sequence."""
    rng = np.random.default_rng(43)
    L, d = 19, 6
    q, k, v = _rand((1, 2, L, d), rng), _rand((1, 2, L, d), rng), _rand((1, 2, L, d), rng)
    o, lse = win(q, k, v, 0.45, 0, -1)
    r = slice(None, None, -1)
    o2, lse2 = ref.attention_f64(q[:, :, r], k[:, :, r], v[:, :, r], 0.45, True)
    np.testing.assert_allclose(o, o2[:, :, r], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2[:, :, r], rtol=0, atol=1e-13)


def pin_closed_forms(win):
    rng = np.random.default_rng(44)
    L, d = 12, 5
    q, k, v = _rand((1, 1, L, d), rng), _rand((1, 1, L, d), rng), _rand((1, 1, L, d), rng)
    # (0, 0): each query sees only its own key
    o, lse = win(q, k, v, 0.3, 0, 0)
    np.testing.assert_allclose(o, v, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], 0.3 * np.einsum("id,id->i", q[0, 0], k[0, 0]), atol=1e-13)
    # K = 0: uniform weights over the window
    for wl, wr in [(2, 1), (0, 3)]:
        o, lse = win(q, np.zeros_like(k), v, 0.3, wl, wr)
        for i in range(L):
            lo, hi = max(0, i - wl), min(L, i + wr + 1)
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, lo:hi].mean(axis=0), atol=1e-13)
            assert lse[0, 0, i] == pytest.approx(math.log(hi - lo), abs=1e-13)
    # rows that see no key: Lq > Lk with a causal-side window
    qq = _rand((1, 1, 10, d), rng)
    o, lse = win(qq, k[:, :, :4], v[:, :, :4], 0.3, 1, 0)
    assert np.all(o[0, 0, 6:] == 0) and np.all(np.isneginf(lse[0, 0, 6:]))
    assert np.all(np.isfinite(lse[0, 0, :5]))


def pin_brute_force(win):
    rng = np.random.default_rng(45)
    for (Lq, Lk) in [(1, 1), (3, 7), (7, 3), (8, 8)]:
        for (wl, wr) in [(0, 0), (1, 0), (0, 1), (2, 3), (-1, 1), (1, -1)]:
            q, k, v = _rand((1, 1, Lq, 3), rng, 0.5), _rand((1, 1, Lk, 3), rng, 0.5), _rand((1, 1, Lk, 3), rng)
            o, lse = win(q, k, v, 0.7, wl, wr)
            m = _visible(Lq, Lk, wl, wr)
            for i in range(Lq):
                vis = np.nonzero(m[i])[0]
                if len(vis) == 0:
                    assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i])
                    continue
                e = [math.exp(0.7 * math.fsum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(3))) for j in vis]
                z = math.fsum(e)
                for t in range(3):
                    assert o[0, 0, i, t] == pytest.approx(math.fsum(w * v[0, 0, j, t] for w, j in zip(e, vis)) / z,
                                                          abs=1e-13)
                assert lse[0, 0, i] == pytest.approx(math.log(z), abs=1e-13)


def pin_sampled_rows(win):
    rng = np.random.default_rng(46)
    q, k, v = _rand((1, 2, 30, 4), rng), _rand((1, 2, 30, 4), rng), _rand((1, 2, 30, 4), rng)
    rows = np.stack([np.sort(rng.choice(30, 7, replace=False)) for _ in range(2)])
    o, lse = win(q, k, v, 0.4, 4, 2)
    os_, ls = win(q, k, v, 0.4, 4, 2, rows=rows)
    for bh in range(2):
        np.testing.assert_allclose(os_[0, bh], o[0, bh, rows[bh]], atol=0)
        np.testing.assert_allclose(ls[0, bh], lse[0, bh, rows[bh]], atol=0)


PINS = [pin_torch_mask, pin_reduces_to_full_and_causal, pin_reversed_causal, pin_closed_forms,
        pin_brute_force, pin_sampled_rows]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_window_oracle_pin(pin):
    pin(ref.attention_window_f64)


MUTANTS = {
    "left_edge_off_by_one": ("(int64_t)i - wl > a) a = (int64_t)i - wl;", "(int64_t)i - wl + 1 > a) a = (int64_t)i - wl + 1;"),
    "right_edge_exclusive": ("b = (int64_t)i + wr + 1;", "b = (int64_t)i + wr;"),
    "bounds_swapped": ("window_range(i, Lk, wl, wr, &lo, &hi);", "window_range(i, Lk, wr, wl, &lo, &hi);"),
    "empty_row_not_cleared": ("                lse[it] = -INFINITY;\n", "                lse[it] = 0.0;\n"),
    "key_offset_dropped": ("const double *key = k + ((size_t)bh * Lk + j) * d;", "const double *key = k + ((size_t)bh * Lk + j - lo) * d;"),
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
    fn = ctypes.CDLL(str(so)).oracle_attention_window_f64
    fn.restype = ctypes.c_int
    fn.argtypes = ref._lib().oracle_attention_window_f64.argtypes
    real = ref._lib()

    class _Shim:
        oracle_attention_f64 = real.oracle_attention_f64
        oracle_attention_window_f64 = fn

    def win(q, k, v, scale, wl, wr, rows=None):
        saved = ref._LIB
        ref._LIB = _Shim
        try:
            return ref.attention_window_f64(q, k, v, scale, wl, wr, rows=rows, nthreads=1)
        finally:
            ref._LIB = saved

    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(win)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
