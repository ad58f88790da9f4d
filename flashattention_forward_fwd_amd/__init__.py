"""FlashAttention-2 forward (and backward) for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library libfa2.so (C ABI in include/fa2.h);
this package only marshals arguments to it.  PyTorch provides device memory
and the stream.

    from flashattention_forward_fwd_amd import forward
    o, lse = forward(q, k, v, causal=True)      # q [B,H,Lq,d], k/v [B,H,Lk,d] on cuda
    dq, dk, dv = backward(q, k, v, o, lse, do, causal=True)
"""
import math

from . import _lib
from ._lib import (FA2_MAX_SPLITS, FA2_STATIC_SCRATCH_BYTES, FA2Error, fa2_bwd, fa2_bwd_dropout,  # noqa: F401
                   fa2_bwd_dropout_f16, fa2_bwd_f16, fa2_bwd_window, fa2_bwd_window_f16, fa2_bwd_workspace_bytes,
                   fa2_check_args, fa2_fwd, fa2_fwd_dropout, fa2_fwd_dropout_f16, fa2_fwd_f16, fa2_fwd_f32,
                   fa2_fwd_splitkv, fa2_fwd_splitkv_f16, fa2_fwd_splitkv_static, fa2_fwd_window,
                   fa2_fwd_window_f16, fa2_merge_partials, fa2_merge_partials_f16, fa2_splitkv_num_splits,
                   fa2_splitkv_workspace_bytes, lib, status_string)

__all__ = ["forward", "backward", "merge_partials", "FA2Error", "status_string", "FA2_MAX_SPLITS",
           "FA2_STATIC_SCRATCH_BYTES", "fa2_check_args", "fa2_splitkv_workspace_bytes", "fa2_splitkv_num_splits",
           "fa2_bwd_workspace_bytes"] + \
    sorted(n for n in _lib.SIGNATURES if n.startswith("fa2_") and n not in ("fa2_status_string",))


def _check_buffer(t, shape, dtype, device, name):
    """A caller-provided output or workspace must be exactly what the kernels will
    write: the library trusts shapes and never sees strides."""
    if not t.is_cuda or t.device != device:
        raise ValueError("%s must be a device tensor on %s" % (name, device))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, not %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _entry(name, dtype):
    """The bf16 entry point `name` or its fp16 twin for torch dtype `dtype`."""
    import torch
    return getattr(_lib, name + ("_f16" if dtype == torch.float16 else ""))


def forward(q, k, v, causal=False, scale=None, out=None, lse=None, num_splits=None, workspace=None,
            window=None, dropout=None):
    """O = softmax(scale * Q K^T [causal]) V and the per-row logsumexp.

    q: [B, H, Lq, d], k and v: [B, H, Lk, d], all bf16, all fp16 or all fp32 CUDA tensors
    (made contiguous).  scale defaults to fp32(1/sqrt(d)).  Returns (o, lse)
    with o like q and lse fp32 [B, H, Lq].  Enqueued on the current stream.

    num_splits (16-bit only): None runs the one-pass kernel; an int runs the
    split-KV path with that many K/V ranges (0: the library picks).  Its
    workspace is allocated here unless a large enough uint8 device tensor is
    given.

    window (16-bit only): (window_left, window_right) runs ``fa2_fwd_window`` --
    key j visible to query i iff i - window_left <= j <= i + window_right, a
    negative bound meaning unbounded; causal must then be False.

    dropout (16-bit only): (p, seed, offset) runs ``fa2_fwd_dropout`` -- each
    probability kept with probability round(256 (1 - p)) / 256 by the Philox
    keep mask of (seed, offset), kept ones scaled up by the inverse; lse is the
    one without dropout.  Pass the same tuple to ``backward``.

    The fp16 twins (``*_f16``) run for float16 tensors.
    """
    import torch

    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors (no CPU path)")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16, all float16 or all float32")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if tuple(k.shape) != (B, H, Lk, d) or tuple(v.shape) != (B, H, Lk, d):
        raise ValueError("k and v must be [B, H, Lk, d] matching q")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty_like(q)
    _check_buffer(out, q.shape, q.dtype, q.device, "out")
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    _check_buffer(lse, (B, H, Lq), torch.float32, q.device, "lse")
    if workspace is not None:
        _check_buffer(workspace, None, None, q.device, "workspace")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    c = int(bool(causal))
    if (dropout is not None or window is not None or num_splits is not None) and q.dtype == torch.float32:
        raise ValueError("dropout, window and num_splits take bfloat16 or float16 tensors")
    if dropout is not None:
        if window is not None or num_splits is not None:
            raise ValueError("dropout takes no window and no num_splits")
        p_drop, seed, offset = dropout
        _entry("fa2_fwd_dropout", q.dtype)(q, k, v, out, lse, B, H, Lq, Lk, d, scale, c, float(p_drop), int(seed),
                                           int(offset), stream)
        return out, lse
    if window is not None:
        if causal or num_splits is not None:
            raise ValueError("window replaces the causal mask (causal=False) and takes no num_splits")
        wl, wr = window
        _entry("fa2_fwd_window", q.dtype)(q, k, v, out, lse, B, H, Lq, Lk, d, scale, int(wl), int(wr), stream)
        return out, lse
    if num_splits is not None:
        need = fa2_splitkv_workspace_bytes(B, H, Lq, Lk, d, c, num_splits)
        if need == 0:
            raise ValueError("sizes or num_splits rejected by fa2_splitkv_workspace_bytes")
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _entry("fa2_fwd_splitkv", q.dtype)(q, k, v, out, lse, B, H, Lq, Lk, d, scale, c, num_splits, workspace,
                                           workspace.numel() * workspace.element_size(), stream)
        return out, lse
    fn = {torch.bfloat16: fa2_fwd, torch.float16: fa2_fwd_f16, torch.float32: fa2_fwd_f32}[q.dtype]
    fn(q, k, v, out, lse, B, H, Lq, Lk, d, scale, c, stream)
    return out, lse


def merge_partials(o_parts, lse_parts, out=None, lse=None, dtype=None):
    """Combine partial results over disjoint key sets (libfa2 ``fa2_merge_partials``).

    o_parts: fp32 [S, ..., d], lse_parts: fp32 [S, ...] (natural-log
    logsumexps, -inf for an empty part) on the device.  Returns (o, lse) with
    o [..., d] in dtype (bfloat16 by default, or float16, or out's dtype) and lse
    fp32 [...].  Enqueued on the current stream.
    """
    import torch

    if not (o_parts.is_cuda and lse_parts.is_cuda):
        raise ValueError("o_parts and lse_parts must be device tensors (no CPU path)")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts and lse_parts must be float32")
    if tuple(o_parts.shape[:-1]) != tuple(lse_parts.shape) or lse_parts.dim() < 2:
        raise ValueError("o_parts must be lse_parts' shape plus a trailing d")
    S, d = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts[0].numel()
    o_parts, lse_parts = o_parts.contiguous(), lse_parts.contiguous()
    if dtype is None:
        dtype = out.dtype if out is not None else torch.bfloat16
    if dtype not in (torch.bfloat16, torch.float16) or (out is not None and out.dtype != dtype):
        raise ValueError("the merged output is bfloat16 or float16")
    if lse_parts.device != o_parts.device:
        raise ValueError("o_parts and lse_parts must be on one device")
    if out is None:
        out = torch.empty(o_parts.shape[1:], dtype=dtype, device=o_parts.device)
    _check_buffer(out, o_parts.shape[1:], dtype, o_parts.device, "out")
    if lse is None:
        lse = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=o_parts.device)
    _check_buffer(lse, lse_parts.shape[1:], torch.float32, o_parts.device, "lse")
    stream = torch.cuda.current_stream(o_parts.device).cuda_stream
    _entry("fa2_merge_partials", dtype)(o_parts, lse_parts, S, rows, d, out, lse, stream)
    return out, lse


def backward(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None,
             window=None, dropout=None):
    """Gradients (dq, dk, dv) of attention for the upstream gradient dout (libfa2 ``fa2_bwd``).

    q, k, v, o, dout: bfloat16 (or all float16) CUDA tensors (q, o, dout [B, H, Lq, d]; k, v
    [B, H, Lk, d]), o and lse (fp32 [B, H, Lq]) as returned by ``forward`` for
    the same q, k, v, causal and scale.  Returns (dq, dk, dv) in q's dtype.  The
    workspace is allocated here unless a large enough uint8 device tensor is
    given.  window: (window_left, window_right) of a ``forward(..., window=...)``
    call runs ``fa2_bwd_window`` (causal must then be False).  dropout: the
    (p, seed, offset) of a ``forward(..., dropout=...)`` call runs
    ``fa2_bwd_dropout``.  float16 tensors run the ``*_f16`` twins.  Enqueued on
    the current stream.
    """
    import torch

    ts = (q, k, v, o, dout)
    if not all(t.is_cuda for t in ts) or not lse.is_cuda:
        raise ValueError("all tensors must be device tensors (no CPU path)")
    if any(t.dtype != q.dtype for t in ts) or q.dtype not in (torch.bfloat16, torch.float16) \
            or lse.dtype != torch.float32:
        raise ValueError("q, k, v, o, dout must be all bfloat16 or all float16, and lse float32")
    if any(t.dim() != 4 for t in ts):
        raise ValueError("q, k, v, o, dout must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if tuple(k.shape) != (B, H, Lk, d) or tuple(v.shape) != (B, H, Lk, d):
        raise ValueError("k and v must be [B, H, Lk, d] matching q")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, H, Lq):
        raise ValueError("o and dout must have q's shape and lse [B, H, Lq]")
    if any(t.device != q.device for t in ts + (lse,)):
        raise ValueError("all tensors must be on one device")
    q, k, v, o, dout, lse = (t.contiguous() for t in (q, k, v, o, dout, lse))
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check_buffer(t, like.shape, like.dtype, q.device, name)
    need = fa2_bwd_workspace_bytes(B, H, Lq)
    if need == 0:
        raise ValueError("sizes rejected by fa2_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_buffer(workspace, None, None, q.device, "workspace")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    nbytes = workspace.numel() * workspace.element_size()
    if dropout is not None:
        if window is not None:
            raise ValueError("dropout takes no window")
        p_drop, seed, offset = dropout
        _entry("fa2_bwd_dropout", q.dtype)(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale,
                                           int(bool(causal)), float(p_drop), int(seed), int(offset), workspace,
                                           nbytes, stream)
        return dq, dk, dv
    if window is not None:
        if causal:
            raise ValueError("window replaces the causal mask (causal=False)")
        _entry("fa2_bwd_window", q.dtype)(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale,
                                          int(window[0]), int(window[1]), workspace, nbytes, stream)
        return dq, dk, dv
    _entry("fa2_bwd", q.dtype)(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, int(bool(causal)),
                               workspace, nbytes, stream)
    return dq, dk, dv
