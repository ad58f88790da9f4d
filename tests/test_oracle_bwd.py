"""Pins for the backward-pass oracle (no GPU).

``ref.attention_bwd_f64`` (the gradients of exact attention, by the chain rule
through the definition) is pinned here to things other than itself: PyTorch's
float64 CPU autograd through its own attention, central finite differences of
the (separately pinned) forward oracle, closed forms, and identities that any
correct gradient satisfies.  ``test_planted_mistakes_are_caught`` plants
plausible mistakes in copies of the C source and checks that the pins catch each.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import torch

from oracle import ref

BWD_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attn_bwd_ref.c")


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _torch_grads(q, k, v, dout, scale, causal):
    """PyTorch float64 CPU autograd through scaled_dot_product_attention (top-left causal)."""
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=bool(causal), scale=float(scale))
    o.backward(torch.tensor(dout))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


# Each pin takes bwd(q, k, v, dout, scale, causal[, rows, keys]) -> (dq, dk, dv)
# and raises AssertionError when the callable is wrong.
def pin_torch_autograd(bwd):
    rng = np.random.default_rng(31)
    for (B, H, Lq, Lk, d, causal) in [(1, 2, 9, 9, 8, True), (2, 1, 7, 13, 16, False),
                                      (1, 1, 13, 6, 4, True), (1, 1, 6, 13, 3, True),
                                      (1, 1, 33, 33, 64, False)]:
        q, k, v = _rand((B, H, Lq, d), rng), _rand((B, H, Lk, d), rng), _rand((B, H, Lk, d), rng)
        dout = _rand((B, H, Lq, d), rng)
        scale = 1 / math.sqrt(d)
        got = bwd(q, k, v, dout, scale, causal)
        want = _torch_grads(q, k, v, dout, scale, causal)
        for g, w in zip(got, want):
            np.testing.assert_allclose(g, w, rtol=0, atol=1e-12)


def pin_finite_differences(bwd):
    """Central differences of sum(O * dO) through the forward oracle, every coordinate."""
    rng = np.random.default_rng(32)
    h = 1e-5
    for (Lq, Lk, d, causal) in [(4, 5, 3, False), (5, 3, 2, True), (3, 3, 4, True)]:
        q, k, v = _rand((1, 1, Lq, d), rng), _rand((1, 1, Lk, d), rng), _rand((1, 1, Lk, d), rng)
        dout = _rand((1, 1, Lq, d), rng)
        scale = 0.7
        dq, dk, dv = bwd(q, k, v, dout, scale, causal)

        def loss(qq, kk, vv):
            o, _ = ref.attention_f64(qq, kk, vv, scale, causal, nthreads=1)
            return float((o * dout).sum())

        for which, x, g in ((0, q, dq), (1, k, dk), (2, v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][idx] += h
                args_m[which][idx] -= h
                fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            np.testing.assert_allclose(g, fd, rtol=0, atol=1e-8)


def pin_closed_forms(bwd):
    rng = np.random.default_rng(33)
    Lq, d = 9, 6
    q, dout = _rand((1, 1, Lq, d), rng), _rand((1, 1, Lq, d), rng)
    # Lk = 1: O = V0 whatever Q and K are -> dQ = dK = 0, dV0 = sum of dO
    k1, v1 = _rand((1, 1, 1, d), rng), _rand((1, 1, 1, d), rng)
    for causal in (False, True):
        dq, dk, dv = bwd(q, k1, v1, dout, 0.5, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-14)
        np.testing.assert_allclose(dk, 0.0, atol=1e-13)
        np.testing.assert_allclose(dv[0, 0, 0], dout[0, 0].sum(axis=0), atol=1e-13)
    # K = 0: uniform weights 1/n_i -> dQ = 0, dV_j = sum over rows i seeing j of dO_i / n_i,
    # dK_j = scale sum_i (1/n_i) (dO_i.v_j - mean over visible j' of dO_i.v_j') q_i
    Lk = 7
    v = _rand((1, 1, Lk, d), rng)
    for causal in (False, True):
        dq, dk, dv = bwd(q, np.zeros((1, 1, Lk, d)), v, dout, 0.5, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-14)
        dv_want = np.zeros((Lk, d))
        dk_want = np.zeros((Lk, d))
        for i in range(Lq):
            n = min(i + 1, Lk) if causal else Lk
            dp = v[0, 0, :n] @ dout[0, 0, i]
            dv_want[:n] += dout[0, 0, i] / n
            dk_want[:n] += 0.5 * np.outer((dp - dp.mean()) / n, q[0, 0, i])
        np.testing.assert_allclose(dv[0, 0], dv_want, atol=1e-13)
        np.testing.assert_allclose(dk[0, 0], dk_want, atol=1e-13)


def pin_identities(bwd):
    rng = np.random.default_rng(34)
    Lq, Lk, d = 11, 8, 5
    q, k, v = _rand((2, 2, Lq, d), rng), _rand((2, 2, Lk, d), rng), _rand((2, 2, Lk, d), rng)
    dout = _rand((2, 2, Lq, d), rng)
    scale = 0.6
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, dout, scale, causal)
        o, _ = ref.attention_f64(q, k, v, scale, causal)
        # O does not change when every key moves by the same vector: sum_j dK_j = 0
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        # rows of P sum to one: sum_j dV_j = sum_i dO_i
        np.testing.assert_allclose(dv.sum(axis=2), dout.sum(axis=2), atol=1e-12)
        # O is linear in V: <dV, V> = <dO, O> per head
        np.testing.assert_allclose((dv * v).sum(axis=(2, 3)), (dout * o).sum(axis=(2, 3)), atol=1e-12)
        # scores depend on Q and K only through q.k: Q -> tQ, K -> K/t changes nothing,
        # so <dQ, Q> = <dK, K> per head
        np.testing.assert_allclose((dq * q).sum(axis=(2, 3)), (dk * k).sum(axis=(2, 3)), atol=1e-12)


def pin_sampled(bwd):
    rng = np.random.default_rng(35)
    Lq, Lk, d = 20, 17, 4
    q, k, v = _rand((2, 2, Lq, d), rng), _rand((2, 2, Lk, d), rng), _rand((2, 2, Lk, d), rng)
    dout = _rand((2, 2, Lq, d), rng)
    rows = np.stack([np.sort(rng.choice(Lq, 6, replace=False)) for _ in range(4)])
    keys = np.stack([np.sort(rng.choice(Lk, 5, replace=False)) for _ in range(4)])
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, dout, 0.4, causal)
        dqs, dks, dvs = bwd(q, k, v, dout, 0.4, causal, rows=rows, keys=keys)
        for bh in range(4):
            b, h = divmod(bh, 2)
            np.testing.assert_allclose(dqs[b, h], dq[b, h, rows[bh]], atol=0)
            np.testing.assert_allclose(dks[b, h], dk[b, h, keys[bh]], atol=0)
            np.testing.assert_allclose(dvs[b, h], dv[b, h, keys[bh]], atol=0)


def pin_window_autograd(bwd):
    """Windows: PyTorch float64 autograd through its attention with a boolean mask
    (rows without a visible key left out of the loss, where torch gives NaN), the
    full / causal cases, and central differences of the window forward oracle."""
    rng = np.random.default_rng(36)
    for (Lq, Lk, d, wl, wr) in [(13, 13, 8, 3, 0), (11, 17, 4, 2, 5), (16, 9, 8, 4, 1), (9, 9, 4, -1, 2),
                                (10, 10, 4, 0, -1), (12, 5, 4, 1, 0)]:
        q, k, v = _rand((1, 2, Lq, d), rng), _rand((1, 2, Lk, d), rng), _rand((1, 2, Lk, d), rng)
        dout = _rand((1, 2, Lq, d), rng)
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        m = np.ones((Lq, Lk), dtype=bool)
        if wl >= 0:
            m &= j >= i - wl
        if wr >= 0:
            m &= j <= i + wr
        live = m.any(axis=1)
        do_live = dout * live[None, None, :, None]           # empty rows carry no gradient
        got = bwd(q, k, v, do_live, 0.5, False, window=(wl, wr))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(m), scale=0.5)
        (o[:, :, torch.from_numpy(live)] * torch.from_numpy(dout)[:, :, torch.from_numpy(live)]).sum().backward()
        for g, w in zip(got, (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())):
            np.testing.assert_allclose(g, w, rtol=0, atol=1e-12)
        # with every row live, empty-row handling aside, the gradients do not depend on dO of empty rows
        got2 = bwd(q, k, v, dout, 0.5, False, window=(wl, wr))
        for g, w in zip(got2, got):
            np.testing.assert_allclose(g, w, rtol=0, atol=1e-12)
    q, k, v = _rand((1, 1, 9, 4), rng), _rand((1, 1, 9, 4), rng), _rand((1, 1, 9, 4), rng)
    dout = _rand((1, 1, 9, 4), rng)
    for causal, win in ((False, (-1, -1)), (True, (-1, 0)), (True, (20, 0))):
        for g, w in zip(bwd(q, k, v, dout, 0.4, False, window=win), bwd(q, k, v, dout, 0.4, causal)):
            np.testing.assert_allclose(g, w, rtol=0, atol=1e-13)
    # central differences of the window forward oracle
    h = 1e-5
    q, k, v = _rand((1, 1, 6, 3), rng), _rand((1, 1, 7, 3), rng), _rand((1, 1, 7, 3), rng)
    dout = _rand((1, 1, 6, 3), rng)
    dq, dk, dv = bwd(q, k, v, dout, 0.6, False, window=(2, 1))

    def loss(qq, kk, vv):
        o, _ = ref.attention_window_f64(qq, kk, vv, 0.6, 2, 1, nthreads=1)
        return float((o * dout).sum())

    for which, x, g in ((0, q, dq), (1, k, dk), (2, v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            a, b = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
            a[which][idx] += h
            b[which][idx] -= h
            fd[idx] = (loss(*a) - loss(*b)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=0, atol=1e-8)


PINS = [pin_torch_autograd, pin_finite_differences, pin_closed_forms, pin_identities, pin_sampled,
        pin_window_autograd]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_bwd_oracle_pin(pin):
    pin(ref.attention_bwd_f64)


def test_bwd_oracle_rejects_bad_arguments():
    q = np.zeros((1, 1, 4, 8)); k = np.zeros((1, 1, 4, 8))
    with pytest.raises(ValueError):
        ref.attention_bwd_f64(q, k, k, q, 1.0, False, rows=np.array([0, 4]))
    with pytest.raises(ValueError):
        ref.attention_bwd_f64(q, k, k, q, 1.0, False, keys=np.array([-1]))


# ----------------------------------------------------- planted mistakes (CPU only)
MUTANTS = {
    "row_term_sign": ("const double ds = p * (dp[j - lo] - Di);", "const double ds = p * (dp[j - lo] + Di);"),
    "row_term_dropped_in_dk": ("const double ds = p * (dd - Drow[bh * Lq + i]);", "const double ds = p * dd;"),
    "dk_scale_dropped": ("dkj[t] += scale * ds * qi[t];", "dkj[t] += ds * qi[t];"),
    "dv_weighted_by_ds": ("dvj[t] += p * doi[t];", "dvj[t] += ds * doi[t];"),
    "key_rows_start_late": ("if (wr >= 0 && (int64_t)j - wr > a) a = (int64_t)j - wr;",
                            "if (wr >= 0 && (int64_t)j - wr + 1 > a) a = (int64_t)j - wr + 1;"),
    "dq_reads_v": ("dqi[t] += scale * ds * Kb[(size_t)j * d + t];", "dqi[t] += scale * ds * Vb[(size_t)j * d + t];"),
    "lse_without_sum": ("lse[it] = hi > lo ? m + log(l) : -INFINITY;", "lse[it] = hi > lo ? m : -INFINITY;"),
    "dp_from_k": ("dd += doi[t] * Vb[(size_t)j * d + t];", "dd += doi[t] * Kb[(size_t)j * d + t];"),
    "causal_ignored_in_rows": ("if (wr >= 0 && (int64_t)i + wr + 1 < b) b = (int64_t)i + wr + 1;",
                               "if (0 && (int64_t)i + wr + 1 < b) b = (int64_t)i + wr + 1;"),
    "window_left_ignored_for_keys": ("if (wl >= 0 && (int64_t)j + wl + 1 < b) b = (int64_t)j + wl + 1;",
                                     "if (0 && (int64_t)j + wl + 1 < b) b = (int64_t)j + wl + 1;"),
}


def _load_mutant(name, tmp_path):
    src = open(BWD_SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src.replace(old, new))
    so = tmp_path / ("mut_%s.so" % name)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    fn = lib.oracle_attention_bwd_f64
    fn.restype = ctypes.c_int
    fn.argtypes = ref._lib().oracle_attention_bwd_f64.argtypes
    fnw = lib.oracle_attention_bwd_window_f64
    fnw.restype = ctypes.c_int
    fnw.argtypes = ref._lib().oracle_attention_bwd_window_f64.argtypes

    class _Shim:
        """The real library for the forward, the mutant for the backward."""
        oracle_attention_f64 = ref._lib().oracle_attention_f64
        oracle_attention_window_f64 = ref._lib().oracle_attention_window_f64
        oracle_attention_bwd_f64 = fn
        oracle_attention_bwd_window_f64 = fnw

    def bwd(q, k, v, dout, scale, causal, rows=None, keys=None, window=None):
        saved = ref._LIB
        ref._LIB = _Shim
        try:
            return ref.attention_bwd_f64(q, k, v, dout, scale, causal, rows=rows, keys=keys, nthreads=1,
                                         window=window)
        finally:
            ref._LIB = saved
    return bwd


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, tmp_path):
    bwd = _load_mutant(name, tmp_path)
    caught = []
    for pin in (pin_torch_autograd, pin_closed_forms, pin_identities, pin_window_autograd):
        try:
            with np.errstate(all="ignore"):
                pin(bwd)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
