"""Integer key-set checks at the workloads' full sizes, on every query row and
every head, in the launch configurations the benchmark times.

With a softmax scale of 1e-30 every score is 0 to float precision, every
weight is exactly 1 and the row sums are exact integers, so exp(lse) is the
number of keys a query attended.  That number has a closed form (digest
"읽기(read) 단계": a query at p reads p-W+1 .. p; plus the sinks of the aionda
page below the window):  |A(i)| = min(i + 1, W) + min(n_sink, max(0, i - W + 1)).
A key read twice, a key skipped, a mis-mapped work item or a wrong slot of the
rolling buffer changes the count.  The values do not matter, so the inputs are
drawn on the device from a seeded generator.
"""
import numpy as np
import pytest
import torch

import sliding_window_gqa_amd as swa
from sliding_window_gqa_amd import synth
from tests.gpu_harness import DEV

pytestmark = pytest.mark.gpu

TINY = 1e-30


def count_closed_form(pos, W, n_sink=0):
    """|A(i)| for the absolute positions `pos` (int64 array)."""
    pos = np.asarray(pos, dtype=np.int64)
    lo = np.maximum(pos - W + 1, 0)
    return np.minimum(pos + 1, W) + np.minimum(n_sink, lo)


def counts_of(lse):
    """exp(lse) rounded to the nearest integer (float64 on the host)."""
    return np.rint(np.exp(lse.detach().to(torch.float64).cpu().numpy())).astype(np.int64)


def rand(shape, gen):
    return torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)


def check(lse_bhn, pos_bn, W, n_sink, what):
    """lse [B][Hq][n] against the closed form at positions pos [B][n]."""
    got = counts_of(lse_bhn)
    want = count_closed_form(pos_bn, W, n_sink)[:, None, :]
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{what}: {len(bad)} wrong counts, first at (seq, head, row) {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]}, want {want[bad[0][0], 0, bad[0][2]]}")


def test_counts_prefill_n8192():
    wl = synth.workload(2)
    print(f"key counts {wl.name}", flush=True)
    N, Hq, Hkv, D, W = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    g = torch.Generator(device=DEV).manual_seed(8002)
    p = swa.make_params(1, Hq, Hkv, D, W, 0, TINY, wl.rope_theta)
    q, k, v = rand((1, N, Hq, D), g), rand((1, N, Hkv, D), g), rand((1, N, Hkv, D), g)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, lse = swa.swa_prefill_chunk(p, q, k, v, None, None, st)
    check(lse, np.arange(N)[None], W, 0, "prefill n8192")


def test_counts_chunked_n16384_and_full_causal():
    wl = synth.workload(3)
    print(f"key counts {wl.name}", flush=True)
    N, Hq, Hkv, D, W, C = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.chunk
    g = torch.Generator(device=DEV).manual_seed(8003)
    p = swa.make_params(1, Hq, Hkv, D, W, 0, TINY, wl.rope_theta)
    q, k, v = rand((1, N, Hq, D), g), rand((1, N, Hkv, D), g), rand((1, N, Hkv, D), g)
    kc = torch.zeros((1, W, Hkv, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    # the chunks through swa_prefill_chunk, then again (fresh caches) through
    # swa_prefill_chunk_aligned: chunks of W tokens from 0, starts multiples of W
    for entry in (swa.swa_prefill_chunk, swa.swa_prefill_chunk_aligned):
        kc.zero_()
        vc.zero_()
        for c in range(N // C):
            s = c * C
            st = torch.tensor([s], dtype=torch.int32, device=DEV)
            qc, kk, vv = (x[:, s:s + C].contiguous() for x in (q, k, v))
            _, lse = entry(p, qc, kk, vv, kc if c else None, vc if c else None, st)
            swa.swa_cache_write(p, kk, vv, st, kc, vc)
            check(lse, np.arange(s, s + C)[None], W, 0, f"{entry.__name__} chunk {c}")
    Wf = wl.extra["full_window"]
    pf = swa.make_params(1, Hq, Hkv, D, Wf, 0, TINY, wl.rope_theta)
    _, lse = swa.swa_prefill_chunk(pf, q, k, v, None, None, torch.zeros(1, dtype=torch.int32, device=DEV))
    check(lse, np.arange(N)[None], Wf, 0, "full causal")


def test_counts_sink_chunk_b16():
    """The sink workload's 4096-token chunk per sequence against its rolling
    cache (4 sinks + 4092 slots), every sequence at its own start."""
    wl = synth.workload(5)
    print(f"key counts {wl.name} chunk", flush=True)
    B, Hq, Hkv, D, W, S, C = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.n_sink, wl.chunk
    g = torch.Generator(device=DEV).manual_seed(8005)
    p = swa.make_params(B, Hq, Hkv, D, W, S, TINY, wl.rope_theta)
    starts = synth.positions(5, B, wl.pos_lo, wl.pos_hi).numpy().astype(np.int64) + 256
    kc = rand((B, S + W, Hkv, D), g)
    vc = rand((B, S + W, Hkv, D), g)
    q, k, v = rand((B, C, Hq, D), g), rand((B, C, Hkv, D), g), rand((B, C, Hkv, D), g)
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    _, lse = swa.swa_prefill_chunk(p, q, k, v, kc, vc, st)
    check(lse, starts[:, None] + np.arange(C)[None], W, S, "sink chunk")


@pytest.mark.parametrize("index", [4, 5])
def test_counts_decode_steps(index):
    """All decode steps of the batched-decode (64 sequences, positions from 1)
    and sink (16 sequences, 4 sinks) workloads, through swa_decode_step as the
    benchmark runs them; every step's count is checked for every sequence and
    head, across the fill point p = W - 1 where it occurs."""
    wl = synth.workload(index)
    print(f"key counts {wl.name} decode", flush=True)
    B, Hq, Hkv, D, W, S = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.n_sink
    g = torch.Generator(device=DEV).manual_seed(8000 + index)
    p = swa.make_params(B, Hq, Hkv, D, W, S, TINY, wl.rope_theta)
    p0 = synth.positions(index, B, wl.pos_lo, wl.pos_hi).numpy().astype(np.int64)
    if index == 4:
        p0[:4] = [1, W - 130, W - 1, 2 * W - 3]   # the fill point and a wrap inside the steps
    kc = rand((B, S + W, Hkv, D), g)
    vc = rand((B, S + W, Hkv, D), g)
    steps = wl.steps
    ws = torch.empty(swa.swa_decode_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    lses = torch.empty((steps, B, Hq), dtype=torch.float32, device=DEV)
    for s in range(steps):
        pos = torch.tensor(p0 + s, dtype=torch.int32, device=DEV)
        swa.swa_decode_step(p, rand((B, Hq, D), g), rand((B, Hkv, D), g), rand((B, Hkv, D), g), kc, vc, pos,
                            out, lses[s], ws)
    got = counts_of(lses)                                               # [steps][B][Hq]
    pos = p0[None, :] + np.arange(steps)[:, None]                       # [steps][B]
    want = count_closed_form(pos, W, S)[:, :, None]
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} wrong counts, first at (step, seq, head) {tuple(bad[0])}"


def count_dilated(pos, W, d):
    """|A(i)| of a dilated window without sinks: the progression i, i-d, ...
    inside the span, min(ceil(W/d), floor(i/d) + 1) keys."""
    pos = np.asarray(pos, dtype=np.int64)
    return np.minimum(-(-W // d), pos // d + 1)


@pytest.mark.parametrize("d", [2, 3])
def test_counts_dilated_prefill_n8192(d):
    """The 8192-token layer with a dilated window (the fast kernel's residue
    classes), one pass from position 0 and a second 1000-token chunk against
    the cache it left, every row and head."""
    wl = synth.workload(2)
    print(f"dilated key counts n8192 d={d}", flush=True)
    N, Hq, Hkv, D, W = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    g = torch.Generator(device=DEV).manual_seed(8100 + d)
    p = swa.make_params(1, Hq, Hkv, D, W, 0, TINY, wl.rope_theta, dilation=d)
    q, k, v = rand((1, N, Hq, D), g), rand((1, N, Hkv, D), g), rand((1, N, Hkv, D), g)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, lse = swa.swa_prefill_chunk(p, q, k, v, None, None, st)
    got = counts_of(lse)
    want = count_dilated(np.arange(N), W, d)[None, None, :]
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} wrong counts, first at (seq, head, row) {tuple(bad[0])}"
    kc = torch.zeros((1, W, Hkv, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    swa.swa_cache_write(p, k, v, st, kc, vc)
    C2 = 1000
    q2, k2, v2 = rand((1, C2, Hq, D), g), rand((1, C2, Hkv, D), g), rand((1, C2, Hkv, D), g)
    _, lse2 = swa.swa_prefill_chunk(p, q2, k2, v2, kc, vc, torch.full((1,), N, dtype=torch.int32, device=DEV))
    got = counts_of(lse2)
    want = count_dilated(N + np.arange(C2), W, d)[None, None, :]
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"chunk 2: {len(bad)} wrong counts, first at (seq, head, row) {tuple(bad[0])}"


def test_counts_dilated_decode_b64():
    """The batched-decode workload's shape with dilation 2: 64 steps of the
    64 sequences through swa_decode_step, every count."""
    wl = synth.workload(4)
    print("dilated key counts decode b64", flush=True)
    B, Hq, Hkv, D, W = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    d = 2
    g = torch.Generator(device=DEV).manual_seed(8104)
    p = swa.make_params(B, Hq, Hkv, D, W, 0, TINY, wl.rope_theta, dilation=d)
    p0 = synth.positions(4, B, wl.pos_lo, wl.pos_hi).numpy().astype(np.int64)
    p0[:3] = [1, W - 40, 2 * W - 3]
    kc, vc = rand((B, W, Hkv, D), g), rand((B, W, Hkv, D), g)
    ws = torch.empty(swa.swa_decode_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    steps = 64
    lses = torch.empty((steps, B, Hq), dtype=torch.float32, device=DEV)
    for s in range(steps):
        pos = torch.tensor(p0 + s, dtype=torch.int32, device=DEV)
        swa.swa_decode_step(p, rand((B, Hq, D), g), rand((B, Hkv, D), g), rand((B, Hkv, D), g), kc, vc, pos,
                            out, lses[s], ws)
    got = counts_of(lses)
    want = count_dilated(p0[None, :] + np.arange(steps)[:, None], W, d)[:, :, None]
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} wrong counts, first at (step, seq, head) {tuple(bad[0])}"
