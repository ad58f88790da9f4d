"""Seeded synthetic inputs for the attention forward pass.

This module draws random numbers and fixes shapes, seeds and row samples; it
contains none of the attention arithmetic.  Both sides of every parity check
(the HIP library and the CPU oracle) receive the tensors it returns.

Recipe (the same everywhere):
  * fp32 iid N(0, 1) from ``numpy.random.default_rng(seed).standard_normal``,
    drawn in the order Q, K, V from one generator;
  * for bf16 (fp16) workloads each tensor is rounded to bfloat16 (IEEE half) with
    round-to-nearest-even (PyTorch's CPU conversion); a Q multiplier (the ragged workload uses 4, a power
    of two) is applied after rounding, so it is exact;
  * scale = fp32(1 / sqrt(d));  layout [B, H, L, d] contiguous.
"""
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Lq: int
    Lk: int
    d: int
    dtype: str          # "fp32" or "bf16" ("fp16" for the half-precision variants)
    causal: bool
    seed: int
    q_mult: float = 1.0

    @property
    def scale(self) -> float:
        return float(np.float32(1.0) / np.sqrt(np.float32(self.d)))

    @property
    def flops(self) -> float:
        """4*B*H*Lq*Lk*d, halved for causal -- the metric's work count."""
        f = 4.0 * self.B * self.H * self.Lq * self.Lk * self.d
        return f / 2 if self.causal else f


# The five synthetic workloads.  Seeds 1..5 in order; the 2048-sequence d=64
# workload runs twice (non-causal, causal) from the same seed.
WORKLOADS = {
    "single_head_L256_d64_fp32": Workload("single_head_L256_d64_fp32", 1, 1, 256, 256, 64, "fp32", False, 1),
    "B4_H16_L2048_d64_bf16": Workload("B4_H16_L2048_d64_bf16", 4, 16, 2048, 2048, 64, "bf16", False, 2),
    "B4_H16_L2048_d64_bf16_causal": Workload("B4_H16_L2048_d64_bf16_causal", 4, 16, 2048, 2048, 64, "bf16", True, 2),
    "B2_H32_L4096_d128_bf16_causal": Workload("B2_H32_L4096_d128_bf16_causal", 2, 32, 4096, 4096, 128, "bf16", True, 3),
    "B1_H16_L16384_d128_bf16_causal": Workload("B1_H16_L16384_d128_bf16_causal", 1, 16, 16384, 16384, 128, "bf16", True, 4),
    "B3_H8_Lq1000_Lk7777_d128_bf16_q4": Workload("B3_H8_Lq1000_Lk7777_d128_bf16_q4", 3, 8, 1000, 7777, 128, "bf16", False, 5, 4.0),
}

HEADLINE = "B2_H32_L4096_d128_bf16_causal"

# The split-KV (FlashDecoding) scenario: one query per head against a long K/V
# cache -- the Q-length-1, 128K-context case of "Flash Attention 全解析（上）"
# sections 4.1 and 4.3.  Same recipe, seed 6.
DECODE_WORKLOADS = {
    "B1_H32_Lq1_Lk131072_d128_bf16_decode":
        Workload("B1_H32_Lq1_Lk131072_d128_bf16_decode", 1, 32, 1, 131072, 128, "bf16", False, 6),
}


def random_qkv(B, H, Lq, Lk, d, dtype="bf16", seed=0, q_mult=1.0):
    """Q [B,H,Lq,d], K and V [B,H,Lk,d] as CPU tensors of the requested dtype."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Lq, d), dtype=np.float32)
    k = rng.standard_normal((B, H, Lk, d), dtype=np.float32)
    v = rng.standard_normal((B, H, Lk, d), dtype=np.float32)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
    tq, tk, tv = (torch.from_numpy(a).to(tdt) for a in (q, k, v))
    if q_mult != 1.0:
        tq = tq * q_mult
    return tq.contiguous(), tk.contiguous(), tv.contiguous()


def random_dout(B, H, Lq, d, dtype="bf16", seed=0):
    """Upstream gradient dO [B,H,Lq,d] for the backward pass: fp32 iid N(0, 1) from its
    own generator (seed sequence [seed, 4], so Q, K, V of the same seed are unchanged),
    rounded to the requested dtype like Q, K, V."""
    rng = np.random.default_rng([seed, 4])
    a = rng.standard_normal((B, H, Lq, d), dtype=np.float32)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
    return torch.from_numpy(a).to(tdt).contiguous()


def workload_inputs(w: Workload):
    return random_qkv(w.B, w.H, w.Lq, w.Lk, w.d, w.dtype, w.seed, w.q_mult)


def sample_rows(Lq, n, seed, forced=(0, 1, 63, 64, 127, 128)):
    """Sorted distinct query indices: the forced tile/diagonal edges that exist
    (plus the last row) and the rest uniform without replacement."""
    forced = sorted({r for r in forced if 0 <= r < Lq} | {Lq - 1})
    if n >= Lq:
        return np.arange(Lq, dtype=np.int64)
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(Lq, dtype=np.int64), np.asarray(forced, dtype=np.int64))
    extra = rng.choice(pool, size=n - len(forced), replace=False)
    return np.sort(np.concatenate([np.asarray(forced, dtype=np.int64), extra]))


def head_row_samples(w: Workload, n, seed_offset=1000):
    """Per-(b,h) row samples [B*H, n]: head h of batch b uses seed w.seed+offset+b*H+h."""
    out = np.empty((w.B * w.H, n), dtype=np.int64)
    for bh in range(w.B * w.H):
        out[bh] = sample_rows(w.Lq, n, w.seed + seed_offset + bh)
    return out
