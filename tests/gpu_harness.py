"""Drives the HIP library and the fp64 oracle through the same operations.

GpuSide holds device caches and calls the C ABI through the binding; OracleSide
holds one oracle.RollingCache per sequence.  Inputs come from the seeded
generators in sliding_window_gqa_amd.synth (CPU), so both sides see the same
bf16-rounded values.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.swa_oracle as so
import sliding_window_gqa_amd as swa

DEV = "cuda"


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


class GpuSide:
    def __init__(self, B, Hq, Hkv, D, W, n_sink=0, theta=10000.0, dtype=torch.bfloat16, scale=0.0,
                 fill=float("nan"), dilation=1):
        self.dtype = dtype
        self.p = swa.make_params(B, Hq, Hkv, D, W, n_sink, scale, theta, dtype, dilation)
        self.p_norope = swa.make_params(B, Hq, Hkv, D, W, n_sink, scale, 0.0, dtype, dilation)
        S = n_sink + W
        self.kc = torch.full((B, S, Hkv, D), fill, dtype=dtype, device=DEV)
        self.vc = torch.full((B, S, Hkv, D), fill, dtype=dtype, device=DEV)
        self.has_cache = False

    def write(self, k, v, start, rope=True):
        st = torch.as_tensor(start, dtype=torch.int32).to(DEV)
        swa.swa_cache_write(self.p if rope else self.p_norope, k.to(DEV), v.to(DEV), st, self.kc, self.vc)
        self.has_cache = True

    def prefill(self, q, k, v, start, use_cache=True):
        st = torch.as_tensor(start, dtype=torch.int32).to(DEV)
        kc = self.kc if (use_cache and self.has_cache) else None
        vc = self.vc if (use_cache and self.has_cache) else None
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        out, lse = swa.swa_prefill_chunk(self.p, qd, kd, vd, kc, vc, st)
        swa.swa_cache_write(self.p, kd, vd, st, self.kc, self.vc)
        self.has_cache = True
        return out, lse

    def decode(self, q, k, v, pos, fused=False):
        """Cache write + decode: two calls, or the one-call swa_decode_step."""
        st = torch.as_tensor(pos, dtype=torch.int32).to(DEV)
        self.has_cache = True
        if fused:
            return swa.swa_decode_step(self.p, q.to(DEV), k.to(DEV), v.to(DEV), self.kc, self.vc, st)
        swa.swa_cache_write(self.p, k.to(DEV)[:, None], v.to(DEV)[:, None], st, self.kc, self.vc)
        return swa.swa_decode(self.p, q.to(DEV), self.kc, self.vc, st)


class OracleSide:
    """One oracle RollingCache per sequence (or per sampled sequence)."""

    def __init__(self, seqs, Hkv, D, W, n_sink=0, theta=10000.0, scale=None, dilation=1):
        self.seqs = list(seqs)
        self.theta = theta
        self.scale = scale
        self.caches = {b: so.RollingCache(Hkv, D, W, n_sink, dilation) for b in self.seqs}

    def write(self, k, v, start, rope=True):
        """k, v: [B][n][Hkv][D] tensors (all sequences); start [B]."""
        for b in self.seqs:
            n = k.shape[1]
            pos = np.arange(int(start[b]), int(start[b]) + n)
            kk = np64(k[b])
            if rope:
                kk = so.rope(kk, pos, self.theta)
            self.caches[b].write(kk, np64(v[b]), pos)

    def prefill(self, q, k, v, start, rows=None):
        """Returns {b: (out [rows][Hq][D], lse [Hq][rows])}."""
        res = {}
        for b in self.seqs:
            res[b] = so.prefill_chunk(self.caches[b], np64(q[b]), np64(k[b]), np64(v[b]), int(start[b]),
                                      self.theta, self.scale, rows=rows)
        return res

    def decode(self, q, k, v, pos, compute=True):
        res = {}
        for b in self.seqs:
            p = int(pos[b])
            if compute:
                res[b] = so.decode_step(self.caches[b], np64(q[b]), np64(k[b]), np64(v[b]), p,
                                        self.theta, self.scale)
            else:  # advance the cache only
                kr = so.rope(np64(k[b])[None], np.array([p]), self.theta)
                self.caches[b].write(kr, np64(v[b])[None], [p])
        return res
