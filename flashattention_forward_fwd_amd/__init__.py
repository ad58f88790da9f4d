"""FlashAttention-2 forward for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library libfa2.so (C ABI in include/fa2.h);
this package only marshals arguments to it.  PyTorch provides device memory
and the stream.

    from flashattention_forward_fwd_amd import forward
    o, lse = forward(q, k, v, causal=True)      # q [B,H,Lq,d], k/v [B,H,Lk,d] on cuda
"""
import math

from ._lib import FA2Error, fa2_check_args, fa2_fwd, fa2_fwd_f32, lib, status_string  # noqa: F401

__all__ = ["forward", "fa2_fwd", "fa2_fwd_f32", "fa2_check_args", "FA2Error", "status_string"]


def forward(q, k, v, causal=False, scale=None, out=None, lse=None):
    """O = softmax(scale * Q K^T [causal]) V and the per-row logsumexp.

    q: [B, H, Lq, d], k and v: [B, H, Lk, d], all bf16 or all fp32 CUDA tensors
    (made contiguous).  scale defaults to fp32(1/sqrt(d)).  Returns (o, lse)
    with o like q and lse fp32 [B, H, Lq].  Enqueued on the current stream.
    """
    import torch

    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors (no CPU path)")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if tuple(k.shape) != (B, H, Lk, d) or tuple(v.shape) != (B, H, Lk, d):
        raise ValueError("k and v must be [B, H, Lk, d] matching q")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    fn = fa2_fwd if q.dtype == torch.bfloat16 else fa2_fwd_f32
    fn(q, k, v, out, lse, B, H, Lq, Lk, d, scale, int(bool(causal)), stream)
    return out, lse
