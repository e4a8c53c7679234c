"""The C ABI called from plain C.  tests/c_abi/swa_c_check (built with gcc by
sliding_window_gqa_amd/build.py; no Python or torch in it) allocates its own
device buffers and runs a prefill chunk without a cache, that chunk's cache
write and three fused decode steps.  Its outputs and final caches must equal,
byte for byte, the same calls made through the Python binding on the same
inputs: both run the library's kernels, so any difference is a marshalling
fault on one side."""
import os
import subprocess

import numpy as np
import pytest
import torch

import sliding_window_gqa_amd as swa
from tests.gpu_harness import DEV

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "swa_c_check")
B, HQ, HKV, D, W, C, STEPS = 2, 8, 2, 128, 128, 200, 3


class Draws:
    """The C program's generator: state = state * 1664525 + 1013904223 (mod
    2^32), value (state >> 8) / 2^24 * 2 - 1 in float32, rounded to bf16."""

    def __init__(self, seed=12345):
        self.s = seed

    def take(self, shape):
        n = int(np.prod(shape))
        vals = np.empty(n, dtype=np.uint32)
        s = self.s
        for i in range(n):
            s = (s * 1664525 + 1013904223) & 0xFFFFFFFF
            vals[i] = s >> 8
        self.s = s
        f = vals.astype(np.float32) * np.float32(1.0 / 16777216.0) * np.float32(2.0) - np.float32(1.0)
        return torch.from_numpy(f).to(torch.bfloat16).reshape(shape).to(DEV)


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().tobytes()


def test_c_program_matches_the_binding(tmp_path):
    assert os.path.exists(EXE), f"{EXE} is missing: build it with `python -m sliding_window_gqa_amd.build`"
    out_file = tmp_path / "c_outputs.bin"
    print("C ABI check: running the plain-C caller", flush=True)
    r = subprocess.run([EXE, str(out_file)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"swa_c_check failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    got = out_file.read_bytes()

    p = swa.make_params(B, HQ, HKV, D, W, 0, 0.0, 10000.0, torch.bfloat16)
    dr = Draws()
    q, k, v = dr.take((B, C, HQ, D)), dr.take((B, C, HKV, D)), dr.take((B, C, HKV, D))
    kc = torch.zeros((B, W, HKV, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    start = torch.zeros(B, dtype=torch.int32, device=DEV)
    out, lse = swa.swa_prefill_chunk(p, q, k, v, None, None, start)
    swa.swa_cache_write(p, k, v, start, kc, vc)
    want = [_bytes(out), _bytes(lse)]
    for s in range(STEPS):
        q1, k1, v1 = dr.take((B, HQ, D)), dr.take((B, HKV, D)), dr.take((B, HKV, D))
        pos = torch.full((B,), C + s, dtype=torch.int32, device=DEV)
        o1, l1 = swa.swa_decode_step(p, q1, k1, v1, kc, vc, pos)
        want += [_bytes(o1), _bytes(l1)]
    want += [_bytes(kc), _bytes(vc)]
    torch.cuda.synchronize()

    names = ["prefill out", "prefill lse"] + [f"step {s} {x}" for s in range(STEPS) for x in ("out", "lse")] + \
            ["k_cache", "v_cache"]
    assert len(got) == sum(len(w) for w in want), (len(got), sum(len(w) for w in want))
    off = 0
    for name, w in zip(names, want):
        assert got[off:off + len(w)] == w, f"{name} differs between the C program and the binding"
        off += len(w)
