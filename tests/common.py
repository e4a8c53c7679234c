"""Shared helpers for the parity tests: tolerances, comparison, and the two
sides of a parity run (the HIP library through its binding, and the fp64
oracle) driven through the same sequence of operations.
"""
from __future__ import annotations

import math

import numpy as np
import torch

# Spec tolerances for bf16 inputs with float32 accumulation against the
# fp64 oracle on the same bf16-rounded inputs.
BF16_ATOL, BF16_RRMS = 2e-2, 5e-3
# float32 path: float32 arithmetic throughout (derived in the design notes).
F32_ATOL, F32_RRMS = 1e-4, 1e-5
# log-sum-exp (natural log): score errors average into it; bf16 rounding of
# q and k moves a unit-variance score by ~2e-3.
BF16_LSE_ATOL, F32_LSE_ATOL = 1e-2, 1e-5


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to(torch.float64).cpu().numpy()
    return np.asarray(t, dtype=np.float64)


def errors(got, ref):
    g, r = to64(got), to64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    d = np.abs(g - r)
    return float(d.max()), float(math.sqrt((d ** 2).sum() / max((r ** 2).sum(), 1e-300)))


def assert_close(got, ref, atol, rrms, what=""):
    assert np.isfinite(to64(got)).all(), f"{what}: non-finite values"
    mx, rr = errors(got, ref)
    assert mx <= atol and rr <= rrms, f"{what}: max-abs {mx:.3e} (<= {atol}), rel-RMS {rr:.3e} (<= {rrms})"
    return mx, rr


def assert_lse(got, ref, atol, what=""):
    g, r = to64(got), to64(ref)
    assert np.isfinite(g).all(), f"{what}: non-finite lse"
    mx = float(np.abs(g - r).max())
    assert mx <= atol, f"{what}: lse max-abs {mx:.3e} (<= {atol})"


def tol(dtype):
    if dtype == torch.float32:
        return F32_ATOL, F32_RRMS, F32_LSE_ATOL
    return BF16_ATOL, BF16_RRMS, BF16_LSE_ATOL


def cuda_available() -> bool:
    return torch.cuda.is_available()
