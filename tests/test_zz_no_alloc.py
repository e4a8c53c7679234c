"""swa_decode_step_noalloc (no workspace: the library's fixed scratch array)
against swa_decode_step with a caller workspace, through the C ABI: calls in a
row on one GPU, each smaller than the one before, every result compared bit
for bit (output, LSE, both caches as bytes).  Both entry points run the same
kernels, so the results must be identical."""
import pytest
import torch

import sliding_window_gqa_amd as swa
from tests.gpu_harness import DEV

pytestmark = pytest.mark.gpu

# (batch, Hq, Hkv, head_dim, window, n_sink, dtype, first position): every
# shape splits the slots over several ranges, so the partials go through the
# scratch array; each call is smaller than the one before it
CALLS = [
    (16, 32, 8, 128, 4092, 4, torch.bfloat16, 70000),    # the sink workload's decode shape
    (2, 8, 2, 128, 300, 2, torch.bfloat16, 1000),
    (2, 4, 1, 64, 100, 0, torch.float32, 37),            # generic kernels
]


def _inputs(B, Hq, Hkv, D, W, S, dtype, p0, gen):
    def r(*shape):
        return torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32).to(dtype)
    q, k, v = r(B, Hq, D), r(B, Hkv, D), r(B, Hkv, D)
    kc, vc = r(B, S + W, Hkv, D), r(B, S + W, Hkv, D)
    pos = (p0 + torch.arange(B, device=DEV) * 13).to(torch.int32)
    return q, k, v, kc, vc, pos


def test_noalloc_decode_step_matches_workspace_version():
    gen = torch.Generator(device=DEV).manual_seed(7777)
    for i, (B, Hq, Hkv, D, W, S, dtype, p0) in enumerate(CALLS):
        print(f"noalloc call {i}: B={B} Hq={Hq} Hkv={Hkv} D={D} W={W} S={S} {dtype}", flush=True)
        p = swa.make_params(B, Hq, Hkv, D, W, S, 0.0, 10000.0, dtype)
        assert swa.swa_decode_workspace_bytes(p) <= swa.swa_noalloc_scratch_bytes()
        q, k, v, kc, vc, pos = _inputs(B, Hq, Hkv, D, W, S, dtype, p0, gen)
        kc2, vc2 = kc.clone(), vc.clone()
        o1 = torch.empty((B, Hq, D), dtype=dtype, device=DEV)
        l1 = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
        swa.swa_decode_step_noalloc(p, q, k, v, kc, vc, pos, o1, l1)
        o2, l2 = swa.swa_decode_step(p, q, k, v, kc2, vc2, pos)
        torch.cuda.synchronize()
        assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"call {i}: outputs differ"
        assert torch.equal(kc.view(torch.uint8), kc2.view(torch.uint8)), f"call {i}: k cache differs"
        assert torch.equal(vc.view(torch.uint8), vc2.view(torch.uint8)), f"call {i}: v cache differs"
