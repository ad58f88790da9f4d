"""Reference implementations in float64 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this module.  The product path never does, and nothing here is
shared with the HIP library.

Three references, each a plain reading of the pages:

* ``attention_f64`` -- the definition of exact attention (scores, three-pass safe
  softmax, P*V, logsumexp), computed by the C library ``liboracle.so`` built from
  ``attn_ref.c`` with the whole score row materialised.
* ``softmax_3pass`` / ``online_softmax`` -- the safe softmax as three passes, and the
  running-max / running-sum recurrence that replaces the first two passes.
* ``flash_attention2_tiled`` -- the blockwise forward (Q blocks outside, K/V blocks
  inside, each block reduced to its own max, sum, normalised output and
  logsumexp, the blocks folded by the rescaling rule of ``merge_partials``), used
  to show on the CPU that the blockwise method reaches the definition's result.
* ``attention_window_f64`` -- the definition restricted to a window of keys around
  each query (sliding-window / local attention), computed by ``attn_window_ref.c``.
* ``philox4x32_10`` / ``dropout_mask`` / ``attention_dropout_f64`` -- the counter-based
  generator of the SC'11 Philox paper, the dropout keep mask drawn from it, and
  attention with dropout on the probabilities (forward and gradients), computed by
  ``attn_dropout_ref.c``.
* ``attention_bwd_f64`` -- the gradients dQ, dK, dV of the definition (the
  backward pass), by the chain rule, computed by ``attn_bwd_ref.c``.
* ``merge_partials`` -- the combine of attention results over disjoint key sets
  from their outputs and logsumexps (ring attention's two-segment merge, and
  FlashDecoding's reduce step).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        lib.oracle_attention_f64.restype = ctypes.c_int
        lib.oracle_attention_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_attention_window_f64.restype = ctypes.c_int
        lib.oracle_attention_window_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_attention_bwd_f64.restype = ctypes.c_int
        lib.oracle_attention_bwd_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_dropout_mask.restype = ctypes.c_int
        lib.oracle_dropout_mask.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p]
        lib.oracle_attention_dropout_f64.restype = ctypes.c_int
        lib.oracle_attention_dropout_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_attention_bwd_window_f64.restype = ctypes.c_int
        lib.oracle_attention_bwd_window_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        _LIB = lib
    return _LIB


def default_threads():
    """OpenMP threads for the oracle: OMP_NUM_THREADS if set, else the usable cores."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def attention_f64(q, k, v, scale, causal, rows=None, nthreads=None):
    """Exact attention in float64 by its definition.

    Follows "Flash Attention 全解析（上）" section 1.2 (S = QK^T, safe softmax in
    three passes, O = PV) and the logsumexp L = m + log(l) of "FlashAttention 怎么做?
    online softmax 怎么更新?" (section "FlashAttention-2 改了什么").

    q: [B, H, Lq, d]; k, v: [B, H, Lk, d] -- any real dtype, widened to float64.
    scale: the scale the device uses (an fp32 value is widened exactly).
    causal: key j visible to query i iff j <= i (top-left alignment).
    rows: None for every query row, else an int array [B*H, n] (or [n], shared by
          every head) of query indices to compute.
    Returns (o, lse): o [B, H, n, d], lse [B, H, n] in float64.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    assert k.shape == (B, H, Lk, d) and v.shape == (B, H, Lk, d)
    if rows is None:
        nr = Lq
        rows_arr = None
    else:
        rows_arr = np.asarray(rows, dtype=np.int64)
        if rows_arr.ndim == 1:
            rows_arr = np.broadcast_to(rows_arr, (B * H, rows_arr.shape[0]))
        rows_arr = np.ascontiguousarray(rows_arr.reshape(B * H, -1), dtype=np.int64)
        nr = rows_arr.shape[1]
    o = np.empty((B, H, nr, d), dtype=np.float64)
    lse = np.empty((B, H, nr), dtype=np.float64)
    if nthreads is None:
        nthreads = default_threads()
    rc = _lib().oracle_attention_f64(
        q.ctypes.data, k.ctypes.data, v.ctypes.data,
        B, H, Lq, Lk, d, float(scale), int(bool(causal)),
        rows_arr.ctypes.data if rows_arr is not None else None, nr,
        o.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention_f64 rejected its arguments (code %d)" % rc)
    return o, lse


def attention_window_f64(q, k, v, scale, window_left, window_right, rows=None, nthreads=None):
    """Exact attention in float64 over a window of keys around each query.

    Key j is visible to query i iff (window_left < 0 or j >= i - window_left) and
    (window_right < 0 or j <= i + window_right); (-1, -1) is full attention and
    (-1, 0) the causal mask.  Rows that see no key get O = 0 and lse = -inf.
    Sliding-window attention is the variant "Flash Attention 全解析（上）" section
    5.3 names; the pages give no formula (the window above is this project's reading).
    Arguments and results otherwise as ``attention_f64``.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    assert k.shape == (B, H, Lk, d) and v.shape == (B, H, Lk, d)
    rows_arr = _index_rows(rows, B * H)
    nr = Lq if rows_arr is None else rows_arr.shape[1]
    o = np.empty((B, H, nr, d))
    lse = np.empty((B, H, nr))
    if nthreads is None:
        nthreads = default_threads()
    rc = _lib().oracle_attention_window_f64(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Lq, Lk, d, float(scale),
        int(window_left), int(window_right),
        rows_arr.ctypes.data if rows_arr is not None else None, nr,
        o.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention_window_f64 rejected its arguments (code %d)" % rc)
    return o, lse


def _index_rows(idx, BH):
    """None, or an int64 [B*H, n] array of indices ([n] is shared by every head)."""
    if idx is None:
        return None
    a = np.asarray(idx, dtype=np.int64)
    if a.ndim == 1:
        a = np.broadcast_to(a, (BH, a.shape[0]))
    return np.ascontiguousarray(a.reshape(BH, -1), dtype=np.int64)


def attention_bwd_f64(q, k, v, dout, scale, causal, rows=None, keys=None, nthreads=None, window=None):
    """Gradients of exact attention in float64: (dq, dk, dv) for the upstream gradient dout.

    The chain rule through the definition computed by ``attention_f64``:
    dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P * (dP - D),
    dQ = scale dS K, dK = scale dS^T Q.  The pages ask the backward to rebuild
    S and P from the inputs and the per-row logsumexp instead of storing them
    ("FlashAttention 怎么做? online softmax 怎么更新?", section "Recomputation");
    they print no gradient formulas, so these are the derivative written out.

    q, dout: [B, H, Lq, d]; k, v: [B, H, Lk, d].  rows / keys: None for all, else
    index arrays [B*H, n] (or [n] shared by every head) selecting the query rows
    of dq and the keys of dk, dv.  window: None, or (window_left, window_right) of
    ``attention_window_f64`` (causal is then ignored); rows that see no key get
    dq = 0 and contribute nothing.  Returns dq [B, H, nr, d], dk, dv [B, H, nk, d].
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    assert k.shape == (B, H, Lk, d) and v.shape == (B, H, Lk, d) and dout.shape == q.shape
    rows_arr = _index_rows(rows, B * H)
    keys_arr = _index_rows(keys, B * H)
    nr = Lq if rows_arr is None else rows_arr.shape[1]
    nk = Lk if keys_arr is None else keys_arr.shape[1]
    dq = np.empty((B, H, nr, d))
    dk = np.empty((B, H, nk, d))
    dv = np.empty((B, H, nk, d))
    if nthreads is None:
        nthreads = default_threads()
    if window is None:
        fn, mask = _lib().oracle_attention_bwd_f64, (int(bool(causal)),)
    else:
        fn, mask = _lib().oracle_attention_bwd_window_f64, (int(window[0]), int(window[1]))
    rc = fn(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
        B, H, Lq, Lk, d, float(scale), *mask,
        rows_arr.ctypes.data if rows_arr is not None else None, nr,
        keys_arr.ctypes.data if keys_arr is not None else None, nk,
        dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention_bwd_f64 rejected its arguments (code %d)" % rc)
    return dq, dk, dv


def softmax_3pass(x):
    """Safe softmax of a 1-D row in three passes: max, sum of exp(x - m), divide.

    "Flash Attention 全解析（上）" section 1.2, the three-pass safe softmax.
    """
    x = np.asarray(x, dtype=np.float64)
    m = -np.inf
    for xi in x:                      # pass 1: running max over the whole row
        m = max(m, xi)
    l = 0.0
    for xi in x:                      # pass 2: denominator with the final max
        l += np.exp(xi - m)
    return np.array([np.exp(xi - m) / l for xi in x])  # pass 3


def online_softmax(x, block=1):
    """Online softmax of a 1-D row, block by block.

    The running max m and the running sum l are updated together; when a block
    raises the max, the old sum is multiplied by exp(m_old - m_new).  A second
    pass divides exp(x - m_final) by l_final.  "Flash Attention 全解析（上）"
    section 2.2.1 (block = 1) and "FlashAttention 怎么做? online softmax 怎么更新?"
    section "Online softmax" (the worked row (1, 3 | 2, 5) uses block = 2).

    Returns (p, trace) where trace[b] = (m, l) after block b.
    """
    x = np.asarray(x, dtype=np.float64)
    m, l = -np.inf, 0.0
    trace = []
    for start in range(0, len(x), block):
        blk = x[start:start + block]
        m_new = max(m, float(blk.max()))
        l = l * np.exp(m - m_new) + float(np.exp(blk - m_new).sum())
        m = m_new
        trace.append((m, l))
    p = np.exp(x - m) / l
    return p, trace


def flash_attention2_tiled(q, k, v, scale, causal, Br, Bc):
    """The blockwise forward for one head in float64: Q blocks of Br rows, K/V blocks
    of Bc rows, no full score row ever formed.

    q: [Lq, d]; k, v: [Lk, d].  Returns (o [Lq, d], lse [Lq]).

    Every (Q block, K/V block) pair is first reduced on its own to the block's
    statistics: its row max m_j, row sum l_j = sum exp(S_j - m_j), its output
    normalised by that sum, O_j = exp(S_j - m_j) V_j / l_j, and its logsumexp
    L_j = m_j + log l_j (L_j = -inf for a row that sees no key of the block).  The
    K/V blocks of a Q block are visited in ascending order, those whose keys are all
    masked for every row of the Q block are skipped (causal), and their results are
    folded with ``merge_partials``.  Folding (L, O) pairs is the running-state update
    of the pages written for normalised parts: multiplying the old sum and output by
    exp(m_old - m_new) and adding the new block is the same as weighting the two
    normalised parts by exp(L_part - L_new) ("FlashAttention 怎么做? online softmax
    怎么更新?", sections "推导 / 关键公式" and "FlashAttention-2 改了什么", and its
    follow-up "多卡(ring attention)怎么合并两段结果?"; the Q loop outside as in
    "FlashAttention-2 算法架构升级" section 二.2).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, d = q.shape
    Lk = k.shape[0]
    o = np.empty((Lq, d))
    lse = np.empty(Lq)
    for i0 in range(0, Lq, Br):
        i1 = min(i0 + Br, Lq)
        qrow = np.arange(i0, i1)
        o_parts, l_parts = [], []
        for j0 in range(0, Lk, Bc):
            if causal and j0 > qrow[-1]:
                break                       # this block and every later one are masked for all rows
            j1 = min(j0 + Bc, Lk)
            S = scale * (q[i0:i1] @ k[j0:j1].T)
            if causal:
                S = np.where(np.arange(j0, j1)[None, :] > qrow[:, None], -np.inf, S)
            m_blk = S.max(axis=1)
            seen = np.isfinite(m_blk)                   # the row sees a key of this block
            shift = np.where(seen, m_blk, 0.0)
            E = np.exp(S - shift[:, None])              # exp(-inf) = 0 on masked keys
            l_blk = np.where(seen, E.sum(axis=1), 1.0)
            o_parts.append((E @ v[j0:j1]) / l_blk[:, None])
            l_parts.append(np.where(seen, m_blk + np.log(l_blk), -np.inf))
        o[i0:i1], lse[i0:i1] = merge_partials(np.stack(o_parts), np.stack(l_parts))
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint key sets into the result over their union.

    o_parts: [S, ..., d], each part's output normalised by its own row sum;
    lse_parts: [S, ...], each part's logsumexp (natural log; -inf where the part
    has no visible key, in which case its output is ignored and may hold anything).
    Returns (o [..., d], lse [...]) in float64.

    Two normalised segments merge as L = log(e^L1 + e^L2) and
    O = e^(L1 - L) O1 + e^(L2 - L) O2 ("FlashAttention 怎么做? online softmax 怎么更新?",
    follow-up "多卡(ring attention)怎么合并两段结果?").  More parts are folded in one
    at a time with the same two-segment step, which is FlashDecoding's reduce over
    its K/V splits ("Flash Attention 全解析（上）" section 4.3).  A row whose parts
    are all empty gets O = 0 and L = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o = np.zeros(o_parts.shape[1:])
    lse = np.full(lse_parts.shape[1:], -np.inf)
    for s in range(o_parts.shape[0]):
        l2 = lse_parts[s]
        o2 = np.where(np.isneginf(l2)[..., None], 0.0, o_parts[s])   # an empty part is not read
        l_new = np.logaddexp(lse, l2)
        seen = ~np.isneginf(l_new)
        safe = np.where(seen, l_new, 0.0)
        w1 = np.where(seen, np.exp(lse - safe), 0.0)
        w2 = np.where(seen, np.exp(l2 - safe), 0.0)
        o = w1[..., None] * o + w2[..., None] * o2
        lse = l_new
    return o, lse


def dropout_threshold(p):
    """Keep threshold t = round(256 (1 - p)) in 1..256: a byte u keeps iff u < t, so the
    keep probability is t / 256 and kept values are scaled by 256 / t."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(min(256, max(1, round(256.0 * (1.0 - p)))))


def philox4x32_10(ctr, key):
    """Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) of a 4-word counter and
    2-word key (uint32 each); returns the 4 output words."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k_ = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    assert c.shape == (4,) and k_.shape == (2,)
    _lib().oracle_philox4x32_10(c.ctypes.data, k_.ctypes.data, out.ctypes.data)
    return out


def dropout_mask(B, H, Lq, Lk, seed, offset, t):
    """Keep mask [B, H, Lq, Lk] (bool) of the dropout reading: byte (j % 4) of word
    (i % 4) of Philox4x32-10 at counter (j / 4, i / 4, b H + h, offset), key
    (seed low, seed high), kept iff below t."""
    m = np.empty((B, H, Lq, Lk), dtype=np.uint8)
    rc = _lib().oracle_dropout_mask(B, H, Lq, Lk, int(seed), int(offset), int(t), m.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_dropout_mask rejected its arguments (code %d)" % rc)
    return m.astype(bool)


def attention_dropout_f64(q, k, v, scale, causal, seed, offset, t, dout=None, nthreads=None):
    """Attention with dropout on the probabilities, in float64, by definition.

    A = P * mask * 256 / t (mask from ``dropout_mask``), O = A V; lse is the
    logsumexp of the scores without dropout.  With dout, also the gradients:
    dV = A^T dO, dA = dO V^T, dP = dA * mask * 256 / t, D = rowsum(A * dA),
    dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q.  The pages list dropout
    among the steps fused into one pass over a score block ("Flash Attention
    全解析（上）" section 2.1.2) without a formula; the mask, threshold and scale
    are this project's reading.  Returns (o, lse) or (o, lse, dq, dk, dv).
    Holds P for every (row, key): small sizes only.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    o = np.empty((B, H, Lq, d))
    lse = np.empty((B, H, Lq))
    grads = None
    dptr = None
    if dout is not None:
        dout = np.ascontiguousarray(dout, dtype=np.float64)
        grads = (np.empty((B, H, Lq, d)), np.empty((B, H, Lk, d)), np.empty((B, H, Lk, d)))
        dptr = dout.ctypes.data
    if nthreads is None:
        nthreads = default_threads()
    rc = _lib().oracle_attention_dropout_f64(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, dptr, B, H, Lq, Lk, d, float(scale), int(bool(causal)),
        int(seed), int(offset), int(t), o.ctypes.data, lse.ctypes.data,
        grads[0].ctypes.data if grads else None, grads[1].ctypes.data if grads else None,
        grads[2].ctypes.data if grads else None, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention_dropout_f64 rejected its arguments (code %d)" % rc)
    return (o, lse) if grads is None else (o, lse) + grads
