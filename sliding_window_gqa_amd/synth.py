"""Seeded synthetic workloads for sliding-window GQA attention.

This module only draws random inputs; it holds none of the attention
arithmetic.  Both the HIP library's callers (tests, benchmark) and the fp64
oracle are fed from it, on the CPU, so the two sides see identical values.

Every tensor is drawn in float32 from N(0, 1) with its own torch.Generator,
seeded from (workload index, tensor tag, sequence index), so that any one
sequence's tensors can be regenerated alone.  bf16 workloads round the draw to
bfloat16 (round-to-nearest-even, torch's conversion) before anything uses it.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "seed_of", "normal", "positions", "workload"]

_TAGS = {
    "q": 1, "k": 2, "v": 3, "pos": 4,
    "hist_k": 5, "hist_v": 6, "garbage_k": 7, "garbage_v": 8,
    "step_q": 9, "step_k": 10, "step_v": 11,
    "sink_k": 12, "sink_v": 13, "chunk_q": 14, "chunk_k": 15, "chunk_v": 16,
    "full_q": 17, "full_k": 18, "full_v": 19,
}


def seed_of(index: int, tag: str, seq: int = 0) -> int:
    """Seed of one tensor: distinct for every (workload, tag, sequence)."""
    return 1000 + index + 1_000_003 * _TAGS[tag] + 7_919 * seq


def normal(shape, index: int, tag: str, seq: int = 0, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0,1) draw in float32 on the CPU, rounded to ``dtype``."""
    g = torch.Generator().manual_seed(seed_of(index, tag, seq))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return x.to(dtype)


def positions(index: int, n: int, lo: int, hi: int) -> torch.Tensor:
    """``n`` integer positions uniform in [lo, hi] (inclusive), int32."""
    g = torch.Generator().manual_seed(seed_of(index, "pos"))
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64).to(torch.int32)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    n_sink: int = 0
    rope_theta: float = 10000.0
    dtype: torch.dtype = torch.bfloat16
    scale: float = 0.0            # 0 means 1/sqrt(head_dim)
    seq_len: int = 0              # prefill tokens
    chunk: int = 0                # chunk length for chunked prefill
    steps: int = 0                # decode steps (per phase for the sink workload)
    pos_lo: int = 0
    pos_hi: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def n_slots(self) -> int:
        return self.n_sink + self.window


# The five workloads: shapes, sizes and value distributions of the pages'
# Mistral-7B attention layer (32 query / 8 KV heads, head_dim 128, W = 4096).
WORKLOADS = {
    1: Workload(1, "tiny_fp32_prefill", batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64,
                window=64, rope_theta=0.0, dtype=torch.float32, scale=0.125, seq_len=256,
                extra={"full_window": 256}),
    2: Workload(2, "prefill_n8192_w4096", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                window=4096, seq_len=8192),
    3: Workload(3, "chunked_prefill_n16384_c4096", batch=1, n_q_heads=32, n_kv_heads=8,
                head_dim=128, window=4096, seq_len=16384, chunk=4096,
                extra={"full_window": 16384}),
    4: Workload(4, "decode_b64_w4096", batch=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
                window=4096, steps=256, pos_lo=1, pos_hi=32768),
    5: Workload(5, "sink_decode_b16_s4_w4092", batch=16, n_q_heads=32, n_kv_heads=8,
                head_dim=128, window=4092, n_sink=4, steps=256, chunk=4096,
                pos_lo=4096, pos_hi=65536),
}


def workload(index: int) -> Workload:
    return WORKLOADS[index]
