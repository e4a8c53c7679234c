"""fp64 CPU oracle for sliding-window GQA attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  See swa_oracle for the
definitions and the readings of the pages they follow.
"""
from .swa_oracle import (  # noqa: F401
    RollingCache,
    decode_step,
    key_mask,
    kv_cache_bytes,
    prefill_chunk,
    rope,
    swa_attention,
)
from .brute import attend_brute, rope_brute  # noqa: F401
