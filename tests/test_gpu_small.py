"""GPU parity on small inputs that still span several tiles and ragged tails:
the HIP library (through the C ABI) against the fp64 oracle, element by
element.  Index work (slots, masks, cache placement) is compared bit-exactly.
"""
import math

import numpy as np
import pytest
import torch

import oracle.swa_oracle as so
import sliding_window_gqa_amd as swa
from sliding_window_gqa_amd import synth
from tests.common import BF16_LSE_ATOL, assert_close, assert_lse, tol
from tests.gpu_harness import DEV, GpuSide, OracleSide, np64

pytestmark = pytest.mark.gpu


def rnd(shape, tag, seq=0, dtype=torch.bfloat16, index=90):
    return synth.normal(shape, index, tag, seq, dtype)


# ---------------------------------------------------------------------------
# integer index work, bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("W,S", [(4096, 0), (4092, 4), (100, 3), (4, 0), (1, 0), (64, 64), (64, 300)])
def test_debug_slots_and_mask_bit_exact(W, S):
    print(f"debug slots/mask W={W} n_sink={S}", flush=True)
    p = swa.make_params(1, 4, 1, 128, W, S)
    g = torch.Generator().manual_seed(W + S)
    pos = torch.cat([torch.arange(0, 300), torch.randint(0, 1 << 24, (500,), generator=g)]).to(torch.int32)
    slots = swa.swa_debug_slots(p, pos.to(DEV)).cpu().numpy()
    cache = so.RollingCache(1, 1, W, S)
    np.testing.assert_array_equal(slots, [cache.slot(int(x)) for x in pos])
    for qp in [0, 1, 3, W - 1, W, W + 1, S + W + 5, 70000]:
        kp = torch.arange(max(0, qp - W - 70), qp + 70, dtype=torch.int32)
        kp = torch.cat([torch.arange(0, S + 3, dtype=torch.int32), kp])
        m = swa.swa_debug_mask(p, qp, kp.to(DEV)).cpu().numpy().astype(bool)
        np.testing.assert_array_equal(m, so.key_mask([qp], kp.numpy(), W, S)[0])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("theta", [0.0, 10000.0])
@pytest.mark.parametrize("S", [0, 3])
def test_cache_write_placement(dtype, theta, S):
    """Slots written must hold exactly the oracle's entries (V verbatim, K
    rotated); slots never written keep their old bytes."""
    print(f"cache write dtype={dtype} theta={theta} n_sink={S}", flush=True)
    B, Hkv, D, W = 3, 2, 128, 20
    gpu = GpuSide(B, 4 * Hkv, Hkv, D, W, S, theta, dtype, fill=7.0)
    orc = OracleSide(range(B), Hkv, D, W, S, theta)
    ops = [(7, [0, 5, 33]), (45, [7, 12, 40]), (1, [52, 57, 85]), (19, [53, 58, 86]), (2, [200, 300, 1000])]
    for n, start in ops:
        k = rnd((B, n, Hkv, D), "k", n, dtype)
        v = rnd((B, n, Hkv, D), "v", n, dtype)
        gpu.write(k, v, start)
        orc.write(k, v, start)
    kc, vc = np64(gpu.kc), np64(gpu.vc)
    for b in range(B):
        c = orc.caches[b]
        held = c.tag >= 0
        np.testing.assert_array_equal(vc[b][held], c.v[held])
        assert (vc[b][~held] == 7.0).all() and (kc[b][~held] == 7.0).all()
        if theta == 0:
            np.testing.assert_array_equal(kc[b][held], c.k[held])
        else:
            err = np.abs(kc[b][held] - c.k[held])
            ulp = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -23
            assert (err <= ulp * np.abs(c.k[held]) + 1e-6).all(), err.max()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("theta", [0.0, 10000.0])
@pytest.mark.parametrize("S", [0, 3])
def test_rope_keys_cache_write_equals_the_two_calls(dtype, theta, S):
    """The one-pass rotation + cache write leaves k_rot and both caches
    byte-identical to swa_rope_keys followed by swa_cache_write: chunks
    shorter and longer than the window, at starts across fills and wraps,
    on NaN-filled caches (a stray store shows)."""
    print(f"rope_keys_cache_write dtype={dtype} theta={theta} n_sink={S}", flush=True)
    B, Hkv, D, W = 3, 2, 128, 20
    p = swa.make_params(B, 4 * Hkv, Hkv, D, W, S, 0.0, theta, dtype)
    for n, start in [(7, [0, 5, 33]), (45, [7, 12, 40]), (1, [52, 57, 85]), (19, [0, 58, 86])]:
        k = rnd((B, n, Hkv, D), "k", n, dtype).to(DEV)
        v = rnd((B, n, Hkv, D), "v", n, dtype).to(DEV)
        st = torch.tensor(start, dtype=torch.int32, device=DEV)
        kc1 = torch.full((B, S + W, Hkv, D), float("nan"), dtype=dtype, device=DEV)
        vc1 = kc1.clone()
        kc2, vc2 = kc1.clone(), vc1.clone()
        kr1 = swa.swa_rope_keys(p, k, st)
        swa.swa_cache_write(p, k, v, st, kc1, vc1)
        kr2 = swa.swa_rope_keys_cache_write(p, k, v, st, kc2, vc2)
        for a, b_, what in ((kr1, kr2, "k_rot"), (kc1, kc2, "k_cache"), (vc1, vc2, "v_cache")):
            assert torch.equal(a.view(torch.uint8), b_.view(torch.uint8)), (what, n, start)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("W", [64, 256])
def test_prefill_tiny_fp32(W):
    """Tiny float32 SWA prefill: batch 1, N=256, 4/1 heads, head_dim 64, no
    RoPE, scale 1/8; W=256 is full causal attention."""
    print(f"tiny fp32 prefill W={W}", flush=True)
    wl = synth.workload(1)
    N, Hq, Hkv, D = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    q = synth.normal((1, N, Hq, D), 1, "q", dtype=torch.float32)
    k = synth.normal((1, N, Hkv, D), 1, "k", dtype=torch.float32)
    v = synth.normal((1, N, Hkv, D), 1, "v", dtype=torch.float32)
    gpu = GpuSide(1, Hq, Hkv, D, W, 0, 0.0, torch.float32, scale=wl.scale)
    orc = OracleSide([0], Hkv, D, W, 0, 0.0, scale=wl.scale)
    out, lse = gpu.prefill(q, k, v, [0])
    ref = orc.prefill(q, k, v, [0])[0]
    atol, rrms, latol = tol(torch.float32)
    assert_close(out[0], ref[0], atol, rrms, "out")
    assert_lse(lse[0], ref[1], latol, "lse")


PREFILL_CASES = [
    # (B, Hq, Hkv, D, W, n_sink, dtype, chunks)  -- fast path: bf16, D=128, groups of 1, 2, 4, 8
    (2, 8, 2, 128, 100, 0, torch.bfloat16, [130, 1, 3, 64, 100, 52]),
    (2, 8, 2, 128, 100, 4, torch.bfloat16, [130, 1, 3, 64, 100, 52]),
    (1, 4, 1, 128, 64, 0, torch.bfloat16, [200, 64, 65]),
    (1, 4, 1, 128, 1, 0, torch.bfloat16, [70, 5]),
    (2, 4, 1, 128, 300, 2, torch.bfloat16, [500, 77]),
    # more (sequence, KV head, query tile) items than CUs: work-groups loop
    # over several items (288 and 272 items in the first and second chunk)
    (2, 32, 8, 128, 300, 0, torch.bfloat16, [1100, 1030]),
    (2, 32, 8, 128, 300, 4, torch.bfloat16, [1100, 1030]),
    # many short items per work-group (2 or 3 tiles each): the tile loads run
    # four tiles ahead across several items (576 and 1032 items)
    (4, 32, 8, 128, 40, 0, torch.bfloat16, [1100, 300]),
    (2, 32, 8, 128, 16, 3, torch.bfloat16, [4100, 50]),
    # a global prefix longer than the window: 4 sink tiles, the last one ragged
    (2, 8, 2, 128, 64, 100, torch.bfloat16, [300, 77, 130]),
    # other group sizes on the fast kernel: 8 (two items per KV head and
    # query tile), 2 and 1 (the item's 4 heads repeat the group's), with and
    # without sinks; Hq < 4 (a query row shorter than an item's 4 heads);
    # more items than CUs
    (2, 16, 2, 128, 100, 0, torch.bfloat16, [130, 1, 3, 64, 100, 52]),
    (2, 16, 2, 128, 100, 4, torch.bfloat16, [130, 1, 64, 52]),
    (2, 4, 2, 128, 100, 0, torch.bfloat16, [130, 1, 3, 64, 52]),
    (2, 4, 2, 128, 100, 3, torch.bfloat16, [130, 1, 64]),
    (2, 2, 2, 128, 100, 0, torch.bfloat16, [130, 1, 64, 52]),
    (1, 1, 1, 128, 64, 2, torch.bfloat16, [200, 65]),
    (1, 2, 1, 128, 64, 0, torch.bfloat16, [200, 65]),
    (2, 64, 8, 128, 300, 0, torch.bfloat16, [1100, 1030]),
    (2, 8, 8, 128, 300, 3, torch.bfloat16, [1100, 70]),
    # generic path
    (2, 4, 2, 64, 100, 0, torch.bfloat16, [130, 1, 70]),
    (1, 6, 2, 128, 50, 3, torch.float32, [90, 7, 40]),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"B{c[0]}H{c[1]}/{c[2]}D{c[3]}W{c[4]}S{c[5]}{str(c[6])[6:]}" for c in PREFILL_CASES])
def test_prefill_chunks(case):
    B, Hq, Hkv, D, W, S, dtype, chunks = case
    print(f"prefill chunks {case}", flush=True)
    theta = 10000.0
    gpu = GpuSide(B, Hq, Hkv, D, W, S, theta, dtype)
    orc = OracleSide(range(B), Hkv, D, W, S, theta)
    # sequence b > 0 starts after a prefix of 237*b tokens already in the cache
    offs = [237 * b for b in range(B)]
    if max(offs) > 0:
        for b in range(1, B):
            pre = 237 * b
            kp = rnd((1, pre, Hkv, D), "hist_k", b, dtype)
            vp = rnd((1, pre, Hkv, D), "hist_v", b, dtype)
            sub = GpuSide(1, Hq, Hkv, D, W, S, theta, dtype)
            sub.write(kp, vp, [0])
            gpu.kc[b] = sub.kc[0]
            gpu.vc[b] = sub.vc[0]
            orc.caches[b].write(so.rope(np64(kp[0]), np.arange(pre), theta), np64(vp[0]), np.arange(pre))
        gpu.has_cache = True
    atol, rrms, latol = tol(dtype)
    t = 0
    for ci, C in enumerate(chunks):
        q = rnd((B, C, Hq, D), "q", ci, dtype)
        k = rnd((B, C, Hkv, D), "k", ci, dtype)
        v = rnd((B, C, Hkv, D), "v", ci, dtype)
        start = [offs[b] + t for b in range(B)]
        out, lse = gpu.prefill(q, k, v, start)
        ref = orc.prefill(q, k, v, start)
        for b in range(B):
            assert_close(out[b], ref[b][0], atol, rrms, f"chunk {ci} seq {b} out")
            assert_lse(lse[b], ref[b][1], latol, f"chunk {ci} seq {b} lse")
        t += C


# (B, Hq, Hkv, D, W, chunk lengths): chunks of W (or 2W) tokens from position
# 0, so every start is a multiple of W; a ragged last chunk
ALIGNED_CASES = [
    (2, 8, 2, 128, 256, [256, 256, 256, 100]),
    (2, 8, 2, 128, 128, [256, 256, 77]),
    (2, 8, 2, 128, 100, [100, 100, 200, 37]),   # a window that is no multiple of the 32-key tile
    (1, 32, 8, 128, 4096, [4096, 4096]),
    (2, 16, 2, 128, 128, [256, 256, 77]),        # groups of 8, 2 and 1
    (2, 4, 2, 128, 100, [100, 100, 37]),
    (2, 2, 2, 128, 128, [128, 128, 50]),
]


@pytest.mark.parametrize("case", ALIGNED_CASES, ids=[f"B{c[0]}H{c[1]}/{c[2]}W{c[4]}" for c in ALIGNED_CASES])
def test_prefill_chunk_aligned(case):
    """swa_prefill_chunk_aligned (the rolling buffer read in slot order) against
    swa_prefill_chunk chunk by chunk: out and LSE byte-identical, with the
    caches written after each chunk; on the small shapes the oracle too.
    Sequence 1 starts one window later than sequence 0 (both multiples of W).
    The caches start as NaN, so a read of a slot not yet written shows."""
    B, Hq, Hkv, D, W, chunks = case
    print(f"prefill chunk aligned {case}", flush=True)
    theta = 10000.0
    gpu = GpuSide(B, Hq, Hkv, D, W, 0, theta)
    small = W <= 256
    orc = OracleSide(range(B), Hkv, D, W, 0, theta) if small else None
    atol, rrms, latol = tol(torch.bfloat16)
    offs = [W * b for b in range(B)]
    t = 0
    for ci, C in enumerate(chunks):
        q, k, v = (rnd((B, C, h, D), n, 300 + ci).to(DEV) for h, n in ((Hq, "q"), (Hkv, "k"), (Hkv, "v")))
        start = [offs[b] + t for b in range(B)]
        st = torch.tensor(start, dtype=torch.int32, device=DEV)
        kc = gpu.kc if gpu.has_cache else None
        vc = gpu.vc if gpu.has_cache else None
        oa, la = swa.swa_prefill_chunk_aligned(gpu.p, q, k, v, kc, vc, st)
        og, lg = swa.swa_prefill_chunk(gpu.p, q, k, v, kc, vc, st)
        torch.cuda.synchronize()
        assert torch.equal(oa.view(torch.int16), og.view(torch.int16)), f"chunk {ci}: out differs"
        assert torch.equal(la.view(torch.int32), lg.view(torch.int32)), f"chunk {ci}: lse differs"
        if orc is not None:
            ref = orc.prefill(q.cpu(), k.cpu(), v.cpu(), start)
            for b in range(B):
                assert_close(oa[b].cpu(), ref[b][0], atol, rrms, f"chunk {ci} seq {b} out")
                assert_lse(la[b].cpu(), ref[b][1], latol, f"chunk {ci} seq {b} lse")
            orc.write(k.cpu(), v.cpu(), start)
        swa.swa_cache_write(gpu.p, k, v, st, gpu.kc, gpu.vc)
        gpu.has_cache = True
        t += C


def test_prefill_chunk_aligned_rejects_a_misaligned_start():
    """A start that is not a multiple of W breaks the entry point's promise:
    that sequence's outputs are all NaN (checked on the device), the other
    sequence's equal swa_prefill_chunk's."""
    B, Hq, Hkv, D, W, C = 2, 8, 2, 128, 128, 100
    print("prefill chunk aligned, misaligned start", flush=True)
    gpu = GpuSide(B, Hq, Hkv, D, W, 0, 10000.0)
    kh, vh = (rnd((B, W, Hkv, D), n, 77).to(DEV) for n in ("hist_k", "hist_v"))   # positions 0 .. W-1
    swa.swa_cache_write(gpu.p, kh, vh, torch.zeros(B, dtype=torch.int32, device=DEV), gpu.kc, gpu.vc)
    q, k, v = (rnd((B, C, h, D), n, 78).to(DEV) for h, n in ((Hq, "q"), (Hkv, "k"), (Hkv, "v")))
    st = torch.tensor([W, W + 5], dtype=torch.int32, device=DEV)   # sequence 1: W + 5 is no multiple
    oa, la = swa.swa_prefill_chunk_aligned(gpu.p, q, k, v, gpu.kc, gpu.vc, st)
    og, lg = swa.swa_prefill_chunk(gpu.p, q, k, v, gpu.kc, gpu.vc, st)
    torch.cuda.synchronize()
    assert torch.equal(oa[0].view(torch.int16), og[0].view(torch.int16))
    assert torch.equal(la[0].view(torch.int32), lg[0].view(torch.int32))
    assert torch.isnan(oa[1].float()).all() and torch.isnan(la[1]).all()
    assert not torch.isnan(og[1].float()).any()


WRITE_PREV_CASES = [(c, 0) for c in ALIGNED_CASES] + [((2, 8, 2, 128, 100, [100, 100, 37]), 3)]


@pytest.mark.parametrize("case,S", WRITE_PREV_CASES, ids=[f"B{c[0]}H{c[1]}/{c[2]}W{c[4]}S{s}" for c, s in WRITE_PREV_CASES])
def test_prefill_chunk_aligned_write_prev(case, S):
    """swa_prefill_chunk_aligned_write_prev (the previous chunk's cache write
    and the next chunk's prefill, the write and the key rotation in one pass)
    against the two calls it replaces, chunk by chunk: out and LSE
    byte-identical, and after the last chunk's own write both caches too.
    With sinks (S = 3) it makes the two calls itself."""
    B, Hq, Hkv, D, W, chunks = case
    print(f"prefill chunk aligned write_prev {case} n_sink={S}", flush=True)
    theta = 10000.0
    one = GpuSide(B, Hq, Hkv, D, W, S, theta)    # the fused entry
    two = GpuSide(B, Hq, Hkv, D, W, S, theta)    # cache write, then the aligned chunk
    offs = [W * b if S == 0 else 0 for b in range(B)]   # with sinks every sequence starts at 0
    t = 0
    prev = None
    for ci, C in enumerate(chunks):
        q, k, v = (rnd((B, C, h, D), n, 400 + ci).to(DEV) for h, n in ((Hq, "q"), (Hkv, "k"), (Hkv, "v")))
        st = torch.tensor([offs[b] + t for b in range(B)], dtype=torch.int32, device=DEV)
        if prev is None:
            o1, l1 = swa.swa_prefill_chunk_aligned(one.p, q, k, v, None, None, st)
            o2, l2 = swa.swa_prefill_chunk_aligned(two.p, q, k, v, None, None, st)
        else:
            kp, vp, sp = prev
            o1, l1 = swa.swa_prefill_chunk_aligned_write_prev(one.p, kp, vp, sp, q, k, v, one.kc, one.vc, st)
            swa.swa_cache_write(two.p, kp, vp, sp, two.kc, two.vc)
            o2, l2 = swa.swa_prefill_chunk_aligned(two.p, q, k, v, two.kc, two.vc, st)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"chunk {ci}: out differs"
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), f"chunk {ci}: lse differs"
        assert not torch.isnan(o1.float()).any(), f"chunk {ci}: NaN (a slot read before it was written)"
        prev = (k, v, st)
        t += C
    for g in (one, two):
        swa.swa_cache_write(g.p, prev[0], prev[1], prev[2], g.kc, g.vc)
    torch.cuda.synchronize()
    assert torch.equal(one.kc.view(torch.int16), two.kc.view(torch.int16))
    assert torch.equal(one.vc.view(torch.int16), two.vc.view(torch.int16))


def test_prefill_chunk_aligned_write_prev_misaligned_start():
    """The fused entry keeps the aligned promise's check: a sequence whose
    next start is no multiple of W gets NaN outputs; the other sequence's
    outputs and both caches equal the two separate calls'."""
    B, Hq, Hkv, D, W, C = 2, 8, 2, 128, 128, 100
    print("prefill chunk aligned write_prev, misaligned start", flush=True)
    one = GpuSide(B, Hq, Hkv, D, W, 0, 10000.0)
    two = GpuSide(B, Hq, Hkv, D, W, 0, 10000.0)
    kp, vp = (rnd((B, W, Hkv, D), n, 79).to(DEV) for n in ("hist_k", "hist_v"))   # positions 0 .. W-1
    sp = torch.zeros(B, dtype=torch.int32, device=DEV)
    q, k, v = (rnd((B, C, h, D), n, 80).to(DEV) for h, n in ((Hq, "q"), (Hkv, "k"), (Hkv, "v")))
    st = torch.tensor([W, W + 5], dtype=torch.int32, device=DEV)
    o1, l1 = swa.swa_prefill_chunk_aligned_write_prev(one.p, kp, vp, sp, q, k, v, one.kc, one.vc, st)
    swa.swa_cache_write(two.p, kp, vp, sp, two.kc, two.vc)
    o2, l2 = swa.swa_prefill_chunk(two.p, q, k, v, two.kc, two.vc, st)
    torch.cuda.synchronize()
    assert torch.equal(o1[0].view(torch.int16), o2[0].view(torch.int16))
    assert torch.equal(l1[0].view(torch.int32), l2[0].view(torch.int32))
    assert torch.isnan(o1[1].float()).all() and torch.isnan(l1[1]).all()
    assert torch.equal(one.kc.view(torch.int16), two.kc.view(torch.int16))
    assert torch.equal(one.vc.view(torch.int16), two.vc.view(torch.int16))


@pytest.mark.parametrize("D,S", [(128, 0), (128, 3), (64, 3)])
def test_prefill_without_cache_at_nonzero_start(D, S):
    """No caches (k_cache = v_cache = NULL) with chunks that start past 0:
    no position before the chunk exists, so the queries attend only the
    chunk's own keys (and the sinks that lie inside the chunk).  The oracle
    sees the same with an empty rolling cache.  D = 128 runs the fast kernel,
    D = 64 the generic one."""
    print(f"prefill without cache, nonzero start, D={D} n_sink={S}", flush=True)
    B, Hq, Hkv, W, theta = 3, 8, 2, 100, 10000.0
    C = 150
    starts = [50, 1000, 2]
    gpu = GpuSide(B, Hq, Hkv, D, W, S, theta)
    orc = OracleSide(range(B), Hkv, D, W, S, theta)
    q = rnd((B, C, Hq, D), "q", 41)
    k = rnd((B, C, Hkv, D), "k", 41)
    v = rnd((B, C, Hkv, D), "v", 41)
    out, lse = gpu.prefill(q, k, v, starts, use_cache=False)
    ref = orc.prefill(q, k, v, starts)
    atol, rrms, latol = tol(torch.bfloat16)
    for b in range(B):
        assert_close(out[b], ref[b][0], atol, rrms, f"seq {b} out")
        assert_lse(lse[b], ref[b][1], latol, f"seq {b} lse")


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (16, 2), (4, 2), (2, 2)])
def test_prefill_key_counts_exact(Hq, Hkv):
    """A (near) zero softmax scale makes every weight exactly 1, so exp(lse)
    counts the keys each query attended: an end-to-end integer check of the
    masks, the window edge, the sinks and the cache/chunk split, for every
    query head (groups of 4, 8, 2 and 1)."""
    print(f"prefill key counts Hq={Hq} Hkv={Hkv}", flush=True)
    B, D, W, S = 2, 128, 100, 4
    gpu = GpuSide(B, Hq, Hkv, D, W, S, 10000.0, torch.bfloat16, scale=1e-30)
    t = 0
    for ci, C in enumerate([150, 70, 1, 130]):
        q = rnd((B, C, Hq, D), "q", ci)
        k = rnd((B, C, Hkv, D), "k", ci)
        v = rnd((B, C, Hkv, D), "v", ci)
        start = [t, t + 1000 * 0]
        _, lse = gpu.prefill(q, k, v, start)
        lse = lse.cpu().numpy()
        for b in range(B):
            for tt in range(C):
                I = start[b] + tt
                count = int(so.key_mask([I], np.arange(I + 1), W, S)[0].sum())
                got = np.rint(np.exp(lse[b, :, tt].astype(np.float64)))
                assert (got == count).all(), (ci, b, tt, got[:4], count)
        t += C


# ---------------------------------------------------------------------------
# dilated windows (the window part keeps keys i, i-d, i-2d, ...)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("W,S,d", [(100, 0, 3), (64, 4, 2), (4096, 0, 2), (300, 100, 5)])
def test_debug_mask_dilated_bit_exact(W, S, d):
    print(f"debug mask W={W} n_sink={S} dilation={d}", flush=True)
    p = swa.make_params(1, 4, 1, 128, W, S, dilation=d)
    for qp in [0, 1, 2, 3, d, W - 1, W, W + 1, S + W + 5, 70001]:
        kp = torch.arange(max(0, qp - W - 70), qp + 70, dtype=torch.int32)
        kp = torch.cat([torch.arange(0, S + 3, dtype=torch.int32), kp])
        m = swa.swa_debug_mask(p, qp, kp.to(DEV)).cpu().numpy().astype(bool)
        np.testing.assert_array_equal(m, so.key_mask([qp], kp.numpy(), W, S, d)[0])


DILATED_PREFILL = [
    # (B, Hq, Hkv, D, W, n_sink, dilation, dtype, chunks) -- without sinks, bf16,
    # head_dim 128 and 4 query heads per KV head: the fast kernel, per residue
    (2, 8, 2, 128, 100, 0, 3, torch.bfloat16, [130, 1, 64, 65, 7]),
    (2, 32, 8, 128, 300, 0, 2, torch.bfloat16, [1100, 1030]),     # several items per work-group
    (1, 4, 1, 128, 4096, 0, 4, torch.bfloat16, [4100, 50]),
    (3, 8, 2, 128, 64, 0, 5, torch.bfloat16, [200, 7, 64]),      # window < 32 * dilation
    (1, 8, 2, 128, 4, 0, 5, torch.bfloat16, [70, 9]),            # dilation > window: only self
    # with sinks, or other shapes: the generic kernel
    (2, 8, 2, 128, 100, 4, 2, torch.bfloat16, [130, 3, 100]),
    (1, 8, 2, 128, 64, 100, 4, torch.bfloat16, [300, 77]),
    (2, 4, 2, 64, 90, 2, 5, torch.bfloat16, [140, 9]),
    (1, 6, 2, 128, 50, 3, 2, torch.float32, [90, 7, 40]),
    (2, 16, 2, 128, 100, 0, 3, torch.bfloat16, [130, 3, 100]),   # a group of 8 (the fast kernel takes 4 dilated)
]


@pytest.mark.parametrize("case", DILATED_PREFILL,
                         ids=[f"B{c[0]}H{c[1]}/{c[2]}D{c[3]}W{c[4]}S{c[5]}d{c[6]}{str(c[7])[6:]}" for c in DILATED_PREFILL])
def test_prefill_dilated(case):
    B, Hq, Hkv, D, W, S, dil, dtype, chunks = case
    print(f"dilated prefill {case}", flush=True)
    theta = 10000.0
    gpu = GpuSide(B, Hq, Hkv, D, W, S, theta, dtype, dilation=dil)
    orc = OracleSide(range(B), Hkv, D, W, S, theta, dilation=dil)
    atol, rrms, latol = tol(dtype)
    offs = [0, 37, 0][:B]
    if B > 1:   # sequence 1 starts after 37 tokens already in its cache
        kp = rnd((1, 37, Hkv, D), "hist_k", 1, dtype)
        vp = rnd((1, 37, Hkv, D), "hist_v", 1, dtype)
        sub = GpuSide(1, Hq, Hkv, D, W, S, theta, dtype, dilation=dil)
        sub.write(kp, vp, [0])
        gpu.kc[1] = sub.kc[0]
        gpu.vc[1] = sub.vc[0]
        gpu.has_cache = True
        orc.caches[1].write(so.rope(np64(kp[0]), np.arange(37), theta), np64(vp[0]), np.arange(37))
    t = 0
    for ci, C in enumerate(chunks):
        q = rnd((B, C, Hq, D), "q", 60 + ci, dtype)
        k = rnd((B, C, Hkv, D), "k", 60 + ci, dtype)
        v = rnd((B, C, Hkv, D), "v", 60 + ci, dtype)
        start = [offs[b] + t for b in range(B)]
        out, lse = gpu.prefill(q, k, v, start)
        ref = orc.prefill(q, k, v, start)
        for b in range(B):
            assert_close(out[b], ref[b][0], atol, rrms, f"chunk {ci} seq {b} out")
            assert_lse(lse[b], ref[b][1], latol, f"chunk {ci} seq {b} lse")
        t += C


@pytest.mark.parametrize("case", [(3, 8, 2, 128, 100, 0, 3, torch.bfloat16), (2, 8, 2, 128, 64, 4, 2, torch.bfloat16),
                                  (2, 4, 1, 64, 100, 2, 4, torch.float32)])
def test_decode_dilated(case):
    """Decode steps through the fill point and wraps, both as cache write +
    decode and as one decode step, against the oracle."""
    B, Hq, Hkv, D, W, S, dil, dtype = case
    print(f"dilated decode {case}", flush=True)
    theta = 10000.0
    gpu = GpuSide(B, Hq, Hkv, D, W, S, theta, dtype, dilation=dil)
    orc = OracleSide(range(B), Hkv, D, W, S, theta, dilation=dil)
    atol, rrms, latol = tol(dtype)
    p0 = [0, 57, 250][:B]
    for b in range(B):
        if p0[b] == 0:
            continue
        kh = rnd((1, p0[b], Hkv, D), "hist_k", 70 + b, dtype)
        vh = rnd((1, p0[b], Hkv, D), "hist_v", 70 + b, dtype)
        sub = GpuSide(1, Hq, Hkv, D, W, S, theta, dtype, dilation=dil)
        sub.write(kh, vh, [0])
        gpu.kc[b] = sub.kc[0]
        gpu.vc[b] = sub.vc[0]
        orc.caches[b].write(so.rope(np64(kh[0]), np.arange(p0[b]), theta), np64(vh[0]), np.arange(p0[b]))
    for st in range(140):
        q = rnd((B, Hq, D), "step_q", 80 + st, dtype)
        k = rnd((B, Hkv, D), "step_k", 80 + st, dtype)
        v = rnd((B, Hkv, D), "step_v", 80 + st, dtype)
        pos = [p0[b] + st for b in range(B)]
        out, lse = gpu.decode(q, k, v, pos, fused=st % 2 == 1)
        ref = orc.decode(q, k, v, pos)
        for b in range(B):
            assert_close(out[b], ref[b][0], atol, rrms, f"step {st} seq {b} out")
            assert_lse(lse[b], ref[b][1], latol, f"step {st} seq {b} lse")


def test_dilated_key_counts_exact():
    """Scale ~ 0: exp(lse) counts the keys; the dilated window holds
    min(ceil(W/d), floor(i/d) + 1) of them, the sinks add those below it."""
    print("dilated key counts", flush=True)
    B, Hq, Hkv, D, W, S, dil = 2, 8, 2, 128, 100, 3, 3
    gpu = GpuSide(B, Hq, Hkv, D, W, S, 10000.0, torch.bfloat16, scale=1e-30, dilation=dil)
    t = 0
    for ci, C in enumerate([150, 70, 1, 130]):
        q = rnd((B, C, Hq, D), "q", 90 + ci)
        k = rnd((B, C, Hkv, D), "k", 90 + ci)
        v = rnd((B, C, Hkv, D), "v", 90 + ci)
        _, lse = gpu.prefill(q, k, v, [t, t])
        lse = lse.cpu().numpy()
        for tt in range(C):
            I = t + tt
            count = int(so.key_mask([I], np.arange(I + 1), W, S, dil)[0].sum())
            got = np.rint(np.exp(lse[:, :, tt].astype(np.float64)))
            assert (got == count).all(), (ci, tt, got.ravel()[:4], count)
        t += C
    for st in range(0, 40):
        pos = [t + st] * B
        _, lse = gpu.decode(rnd((B, Hq, D), "step_q", st), rnd((B, Hkv, D), "step_k", st),
                            rnd((B, Hkv, D), "step_v", st), pos)
        count = int(so.key_mask([t + st], np.arange(t + st + 1), W, S, dil)[0].sum())
        got = np.rint(np.exp(lse.cpu().numpy().astype(np.float64)))
        assert (got == count).all(), (st, got.ravel()[:4], count)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
DECODE_CASES = [
    (3, 8, 2, 128, 100, 0, torch.bfloat16),
    (3, 8, 2, 128, 100, 3, torch.bfloat16),
    (2, 4, 1, 128, 4092, 4, torch.bfloat16),
    (3, 4, 2, 64, 100, 0, torch.bfloat16),   # generic path
    (2, 4, 1, 64, 100, 2, torch.float32),    # generic path
    (2, 8, 2, 128, 64, 100, torch.bfloat16),  # a global prefix longer than the window
    # 16 (sequence, KV head) units x 16 ranges of 384 slots: at most one
    # work-group per CU, so the fast kernel runs 8 waves per work-group
    (2, 32, 8, 128, 4096, 2, torch.bfloat16),
    # other group sizes on the fast kernel: 1 (one query head per KV head),
    # 2 with sinks, 8 over a full 4096-slot window
    (3, 2, 2, 128, 100, 0, torch.bfloat16),
    (2, 4, 2, 128, 300, 3, torch.bfloat16),
    (2, 16, 2, 128, 4096, 0, torch.bfloat16),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"B{c[0]}H{c[1]}/{c[2]}D{c[3]}W{c[4]}S{c[5]}{str(c[6])[6:]}" for c in DECODE_CASES])
def test_decode_steps(case):
    B, Hq, Hkv, D, W, S, dtype = case
    print(f"decode steps {case}", flush=True)
    theta = 10000.0
    gpu = GpuSide(B, Hq, Hkv, D, W, S, theta, dtype)
    orc = OracleSide(range(B), Hkv, D, W, S, theta)
    p0 = [0, 57, 250][:B] if W < 1000 else [3, 5000][:B]
    # history: positions max(0, p0 - W - S) .. p0 - 1, one write per sequence
    for b in range(B):
        lo = max(0, p0[b] - W - S)
        n = p0[b] - lo
        if n == 0:
            continue
        kh = rnd((1, n, Hkv, D), "hist_k", b, dtype)
        vh = rnd((1, n, Hkv, D), "hist_v", b, dtype)
        sub = GpuSide(1, Hq, Hkv, D, W, S, theta, dtype)
        sub.write(kh, vh, [lo])
        orc.caches[b].write(so.rope(np64(kh[0]), np.arange(lo, p0[b]), theta), np64(vh[0]), np.arange(lo, p0[b]))
        if S > 0 and lo > 0:  # sinks of this sequence, written after the history on both sides
            ks = rnd((1, S, Hkv, D), "sink_k", b, dtype)
            vs = rnd((1, S, Hkv, D), "sink_v", b, dtype)
            sub.write(ks, vs, [0])
            orc.caches[b].write(so.rope(np64(ks[0]), np.arange(S), theta), np64(vs[0]), np.arange(S))
        gpu.kc[b] = sub.kc[0]
        gpu.vc[b] = sub.vc[0]
    atol, rrms, latol = tol(dtype)
    steps = 130 if W < 1000 else 40
    for st in range(steps):
        q = rnd((B, Hq, D), "step_q", st, dtype)
        k = rnd((B, Hkv, D), "step_k", st, dtype)
        v = rnd((B, Hkv, D), "step_v", st, dtype)
        pos = [p0[b] + st for b in range(B)]
        out, lse = gpu.decode(q, k, v, pos)
        ref = orc.decode(q, k, v, pos)
        for b in range(B):
            assert_close(out[b], ref[b][0], atol, rrms, f"step {st} seq {b} out")
            assert_lse(lse[b], ref[b][1], latol, f"step {st} seq {b} lse")


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"B{c[0]}H{c[1]}/{c[2]}D{c[3]}W{c[4]}S{c[5]}{str(c[6])[6:]}" for c in DECODE_CASES])
def test_decode_step_fused(case):
    """swa_decode_step against the oracle, and bit for bit against the cache
    write + decode pair it replaces (outputs, LSE and both caches), from the
    first position through the buffer's wrap."""
    B, Hq, Hkv, D, W, S, dtype = case
    print(f"fused decode step {case}", flush=True)
    theta = 10000.0
    one = GpuSide(B, Hq, Hkv, D, W, S, theta, dtype)
    two = GpuSide(B, Hq, Hkv, D, W, S, theta, dtype)
    orc = OracleSide(range(B), Hkv, D, W, S, theta)
    atol, rrms, latol = tol(dtype)
    p0 = [0, 40, 5][:B] if W < 1000 else [4090, 0][:B]
    steps = 120 if W < 1000 else 12
    for st in range(steps):
        q = rnd((B, Hq, D), "step_q", st, dtype, index=91)
        k = rnd((B, Hkv, D), "step_k", st, dtype, index=91)
        v = rnd((B, Hkv, D), "step_v", st, dtype, index=91)
        pos = [p0[b] + st for b in range(B)]
        if st == 0:   # earlier positions of the sequences that do not start at 0
            for b in range(B):
                if p0[b] == 0:
                    continue
                kh = rnd((1, p0[b], Hkv, D), "hist_k", b, dtype, index=91)
                vh = rnd((1, p0[b], Hkv, D), "hist_v", b, dtype, index=91)
                for side in (one, two):
                    sub = GpuSide(1, Hq, Hkv, D, W, S, theta, dtype)
                    sub.write(kh, vh, [0])
                    side.kc[b] = sub.kc[0]
                    side.vc[b] = sub.vc[0]
                orc.caches[b].write(so.rope(np64(kh[0]), np.arange(p0[b]), theta), np64(vh[0]), np.arange(p0[b]))
        o1, l1 = one.decode(q, k, v, pos, fused=True)
        o2, l2 = two.decode(q, k, v, pos)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"step {st}: fused and two-call results differ"
        # as bytes: slots never written hold the same NaN fill on both sides
        assert torch.equal(one.kc.view(torch.uint8), two.kc.view(torch.uint8)), f"step {st} k cache"
        assert torch.equal(one.vc.view(torch.uint8), two.vc.view(torch.uint8)), f"step {st} v cache"
        if st % 7 == 0 or st == steps - 1:
            ref = orc.decode(q, k, v, pos)
            for b in range(B):
                assert_close(o1[b], ref[b][0], atol, rrms, f"step {st} seq {b} out")
                assert_lse(l1[b], ref[b][1], latol, f"step {st} seq {b} lse")
        else:
            orc.decode(q, k, v, pos, compute=False)


def test_decode_key_counts_exact():
    print("decode key counts", flush=True)
    B, Hq, Hkv, D, W, S = 3, 8, 2, 128, 100, 3
    gpu = GpuSide(B, Hq, Hkv, D, W, S, 10000.0, torch.bfloat16, scale=1e-30)
    for st in range(0, 230):
        q = rnd((B, Hq, D), "step_q", st)
        k = rnd((B, Hkv, D), "step_k", st)
        v = rnd((B, Hkv, D), "step_v", st)
        pos = [st, st, st]
        _, lse = gpu.decode(q, k, v, pos)
        count = int(so.key_mask([st], np.arange(st + 1), W, S)[0].sum())
        got = np.rint(np.exp(lse.cpu().numpy().astype(np.float64)))
        assert (got == count).all(), (st, got.ravel()[:4], count)


# ---------------------------------------------------------------------------
# determinism and resume
# ---------------------------------------------------------------------------
def test_bitwise_determinism_and_resume():
    print("determinism and resume", flush=True)
    B, Hq, Hkv, D, W, S = 2, 8, 2, 128, 100, 2
    gpu = GpuSide(B, Hq, Hkv, D, W, S)
    q = rnd((B, 300, Hq, D), "q", 1)
    k = rnd((B, 300, Hkv, D), "k", 1)
    v = rnd((B, 300, Hkv, D), "v", 1)
    st = torch.tensor([0, 0], dtype=torch.int32, device=DEV)
    o1, l1 = swa.swa_prefill_chunk(gpu.p, q.to(DEV), k.to(DEV), v.to(DEV), None, None, st)
    o2, l2 = swa.swa_prefill_chunk(gpu.p, q.to(DEV), k.to(DEV), v.to(DEV), None, None, st)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    gpu.write(k, v, [0, 0])
    steps = []
    for s in range(20):
        steps.append((rnd((B, Hq, D), "step_q", s), rnd((B, Hkv, D), "step_k", s), rnd((B, Hkv, D), "step_v", s)))
    for s in range(10):
        gpu.decode(*steps[s], [300 + s] * B)
    snap = (gpu.kc.clone(), gpu.vc.clone())
    first = [gpu.decode(*steps[s], [300 + s] * B) for s in range(10, 20)]
    gpu.kc.copy_(snap[0])
    gpu.vc.copy_(snap[1])
    second = [gpu.decode(*steps[s], [300 + s] * B) for s in range(10, 20)]
    for (a, la), (b, lb) in zip(first, second):
        assert torch.equal(a, b) and torch.equal(la, lb)


# ---------------------------------------------------------------------------
# varlen batches: chunks of their own lengths, packed
# ---------------------------------------------------------------------------
def _varlen_lens_starts(B, seed):
    g = np.random.default_rng(seed)
    lens = [int(x) for x in np.where(g.random(B) < 0.2, g.integers(20, 90, B), 1)]
    starts = [int(x) for x in g.integers(0, 200, B)]
    return lens, starts


VARLEN_CASES = [
    # B, Hq, Hkv, D, W, sinks, dtype, chunk lengths, start positions
    (5, 8, 2, 128, 100, 3, torch.bfloat16, [0, 1, 130, 64, 7], [0, 250, 40, 0, 300]),
    (4, 8, 2, 128, 4096, 0, torch.bfloat16, [300, 1, 65, 129], [0, 70, 3, 0]),
    (3, 4, 1, 64, 100, 0, torch.float32, [3, 0, 70], [10, 5, 0]),       # generic path
    (70, 8, 2, 128, 64, 0, torch.bfloat16) + _varlen_lens_starts(70, 7),  # two launches, mixed with decodes
    # chunks of one length in one contiguous run per group of 64 sequences
    # (the step takes the fixed-length kernels for the run): sinks, a wrap,
    # empty and one-token sequences on both sides of the run
    (6, 8, 2, 128, 100, 3, torch.bfloat16, [1, 96, 96, 96, 1, 0], [40, 250, 0, 130, 7, 9]),
    (4, 8, 2, 128, 4096, 0, torch.bfloat16, [129, 129, 1, 1], [0, 5000, 70, 4095]),
    (70, 8, 2, 128, 64, 0, torch.bfloat16, [1] * 10 + [70] * 5 + [1] * 49 + [33] * 3 + [1] * 3,
     [int(x) for x in np.random.default_rng(8).integers(0, 200, 70)]),
    # 16 one-token sequences x 8 KV heads x 2 ranges: the step's decode runs
    # 8 waves per work-group (one per CU) through the sequence map
    (17, 32, 8, 128, 4096, 0, torch.bfloat16, [1] * 16 + [100], [4100 + 61 * b for b in range(16)] + [4096]),
    # other group sizes (8, 2, 1) through the varlen kernels and the mixed step
    (5, 16, 2, 128, 100, 3, torch.bfloat16, [0, 1, 130, 64, 7], [0, 250, 40, 0, 300]),
    (4, 4, 2, 128, 4096, 0, torch.bfloat16, [300, 1, 65, 129], [0, 70, 3, 0]),
    (6, 2, 2, 128, 100, 3, torch.bfloat16, [1, 96, 96, 96, 1, 0], [40, 250, 0, 130, 7, 9]),
    (4, 16, 2, 128, 4096, 0, torch.bfloat16, [129, 129, 1, 1], [0, 5000, 70, 4095]),
    # a run longer than the window (only its last W tokens reach the cache)
    # whose write rides on the one-split decode launch
    (5, 8, 2, 128, 64, 0, torch.bfloat16, [1, 100, 100, 1, 1], [30, 200, 0, 64, 7]),
]


def _varlen_setup(case):
    """Caches holding every position before each sequence's start (GPU and
    oracle), and the packed chunks."""
    B, Hq, Hkv, D, W, S, dtype, lens, starts = case
    theta = 10000.0
    gpu = GpuSide(B, Hq, Hkv, D, W, S, theta, dtype)
    orc = OracleSide(range(B), Hkv, D, W, S, theta)
    for b in range(B):
        if starts[b] == 0:
            continue
        kh = rnd((1, starts[b], Hkv, D), "hist_k", b, dtype, index=92)
        vh = rnd((1, starts[b], Hkv, D), "hist_v", b, dtype, index=92)
        sub = GpuSide(1, Hq, Hkv, D, W, S, theta, dtype)
        sub.write(kh, vh, [0])
        gpu.kc[b] = sub.kc[0]
        gpu.vc[b] = sub.vc[0]
        orc.caches[b].write(so.rope(np64(kh[0]), np.arange(starts[b]), theta), np64(vh[0]), np.arange(starts[b]))
    T = sum(lens)
    q = rnd((T, Hq, D), "chunk_q", 0, dtype, index=92)
    k = rnd((T, Hkv, D), "chunk_k", 0, dtype, index=92)
    v = rnd((T, Hkv, D), "chunk_v", 0, dtype, index=92)
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    return gpu, orc, q, k, v, st


VARLEN_IDS = [f"B{c[0]}H{c[1]}/{c[2]}D{c[3]}W{c[4]}S{c[5]}{str(c[6])[6:]}" for c in VARLEN_CASES]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=VARLEN_IDS)
def test_prefill_varlen(case):
    """Packed chunks of different lengths (length 1 = a decode token) against
    the oracle per sequence, and bit for bit against each sequence alone
    through the fixed-length calls: attention output, LSE and the cache write."""
    B, Hq, Hkv, D, W, S, dtype, lens, starts = case
    print(f"varlen prefill B={B} lens={lens[:8]} starts={starts[:8]}", flush=True)
    theta = 10000.0
    gpu, orc, q, k, v, st = _varlen_setup(case)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = swa.swa_prefill_chunk_varlen(gpu.p, qd, kd, vd, gpu.kc, gpu.vc, st, lens)
    p1 = swa.make_params(1, Hq, Hkv, D, W, S, 0.0, theta, dtype)
    atol, rrms, latol = tol(dtype)
    r = 0
    for b in range(B):
        n = lens[b]
        if n == 0:
            continue
        o1, l1 = swa.swa_prefill_chunk(p1, qd[r:r + n][None].contiguous(), kd[r:r + n][None].contiguous(),
                                       vd[r:r + n][None].contiguous(), gpu.kc[b:b + 1], gpu.vc[b:b + 1],
                                       st[b:b + 1])
        assert torch.equal(o1[0], out[r:r + n]), f"seq {b}: varlen output differs from the fixed-length call"
        assert torch.equal(l1[0], lse[:, r:r + n]), f"seq {b}: varlen LSE differs from the fixed-length call"
        if b < 12 or n > 1:   # the oracle on every chunk and the first decode-like rows
            ro, rl = so.prefill_chunk(orc.caches[b], np64(q[r:r + n]), np64(k[r:r + n]), np64(v[r:r + n]),
                                      starts[b], theta)
            assert_close(out[r:r + n].cpu(), ro, atol, rrms, f"seq {b} out")
            assert_lse(lse[:, r:r + n].cpu(), rl, latol, f"seq {b} lse")
        r += n
    # the cache write of the packed chunks = each sequence's own write, byte for byte
    ref_k, ref_v = gpu.kc.clone(), gpu.vc.clone()
    swa.swa_cache_write_varlen(gpu.p, kd, vd, st, lens, gpu.kc, gpu.vc)
    r = 0
    for b in range(B):
        n = lens[b]
        if n:
            swa.swa_cache_write(p1, kd[r:r + n][None].contiguous(), vd[r:r + n][None].contiguous(), st[b:b + 1],
                                ref_k[b:b + 1], ref_v[b:b + 1])
        r += n
    assert torch.equal(gpu.kc.view(torch.uint8), ref_k.view(torch.uint8))
    assert torch.equal(gpu.vc.view(torch.uint8), ref_v.view(torch.uint8))


@pytest.mark.parametrize("case", VARLEN_CASES, ids=VARLEN_IDS)
def test_step_varlen(case):
    """A whole mixed step (one-token sequences through the decode kernel)
    against the oracle per sequence; chunks of more than one token bit for bit
    against swa_prefill_chunk_varlen; the caches afterwards byte for byte
    against swa_cache_write_varlen."""
    B, Hq, Hkv, D, W, S, dtype, lens, starts = case
    print(f"varlen step B={B} lens={lens[:8]} starts={starts[:8]}", flush=True)
    theta = 10000.0
    gpu, orc, q, k, v, st = _varlen_setup(case)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ref_o, ref_l = swa.swa_prefill_chunk_varlen(gpu.p, qd, kd, vd, gpu.kc, gpu.vc, st, lens)
    ref_k, ref_v = gpu.kc.clone(), gpu.vc.clone()
    swa.swa_cache_write_varlen(gpu.p, kd, vd, st, lens, ref_k, ref_v)
    kc0, vc0 = gpu.kc.clone(), gpu.vc.clone()
    out, lse = swa.swa_step_varlen(gpu.p, qd, kd, vd, gpu.kc, gpu.vc, st, lens)
    assert torch.equal(gpu.kc.view(torch.uint8), ref_k.view(torch.uint8))
    assert torch.equal(gpu.vc.view(torch.uint8), ref_v.view(torch.uint8))
    # without an LSE the step writes the same outputs and caches
    out2, lse2 = swa.swa_step_varlen(gpu.p, qd, kd, vd, kc0, vc0, st, lens, want_lse=False)
    assert lse2 is None and torch.equal(out2, out)
    assert torch.equal(kc0.view(torch.uint8), ref_k.view(torch.uint8))
    assert torch.equal(vc0.view(torch.uint8), ref_v.view(torch.uint8))
    atol, rrms, latol = tol(dtype)
    r = 0
    for b in range(B):
        n = lens[b]
        if n == 0:
            continue
        if n > 1:
            assert torch.equal(out[r:r + n], ref_o[r:r + n]) and torch.equal(lse[:, r:r + n], ref_l[:, r:r + n]), b
        ro, rl = so.prefill_chunk(orc.caches[b], np64(q[r:r + n]), np64(k[r:r + n]), np64(v[r:r + n]),
                                  starts[b], theta)
        assert_close(out[r:r + n].cpu(), ro, atol, rrms, f"seq {b} out")
        assert_lse(lse[:, r:r + n].cpu(), rl, latol, f"seq {b} lse")
        r += n


def test_decode_step_graph_replay():
    """Decode steps captured in a HIP graph (the library allocates nothing
    and records no memset): every replay, started from the caches the eager
    steps started from (restored by eager copies between replays, with a
    synchronisation), reproduces the eager outputs, LSE and caches bit for
    bit."""
    print("decode step graph replay", flush=True)
    B, Hq, Hkv, D, W, S = 3, 8, 2, 128, 100, 2
    gpu = GpuSide(B, Hq, Hkv, D, W, S)
    hist = rnd((B, 150, Hkv, D), "hist_k", 0), rnd((B, 150, Hkv, D), "hist_v", 0)
    gpu.write(hist[0], hist[1], [0] * B)
    steps = [(rnd((B, Hq, D), "step_q", s, index=93).to(DEV), rnd((B, Hkv, D), "step_k", s, index=93).to(DEV),
              rnd((B, Hkv, D), "step_v", s, index=93).to(DEV),
              torch.tensor([150 + s, 160 + s, 170 + s], dtype=torch.int32, device=DEV)) for s in range(6)]
    kc0, vc0 = gpu.kc.clone(), gpu.vc.clone()
    ws = torch.empty(swa.swa_decode_workspace_bytes(gpu.p), dtype=torch.uint8, device=DEV)
    eager = [swa.swa_decode_step(gpu.p, q, k, v, gpu.kc, gpu.vc, pos, workspace=ws) for q, k, v, pos in steps]
    kc_e, vc_e = gpu.kc.clone(), gpu.vc.clone()
    outs = [(torch.empty_like(o), torch.empty_like(l)) for o, l in eager]
    gpu.kc.copy_(kc0)
    gpu.vc.copy_(vc0)

    def run():
        for (q, k, v, pos), (o, l) in zip(steps, outs):
            swa.swa_decode_step(gpu.p, q, k, v, gpu.kc, gpu.vc, pos, o, l, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        gpu.kc.copy_(kc0)
        gpu.vc.copy_(vc0)
        for o, l in outs:
            o.zero_()
            l.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for s, ((o, l), (eo, el)) in enumerate(zip(outs, eager)):
            assert torch.equal(o, eo) and torch.equal(l, el), f"replay {rep} step {s}"
        assert torch.equal(gpu.kc.view(torch.uint8), kc_e.view(torch.uint8)), f"replay {rep} k cache"
        assert torch.equal(gpu.vc.view(torch.uint8), vc_e.view(torch.uint8)), f"replay {rep} v cache"
        _ = (gpu.kc.float().sum() + 1).item()   # eager work between replays


def test_first_chunk_and_mixed_step_graph_replay():
    """A first chunk (one-pass rotation + cache write, then attention
    without the cache) and a mixed step whose chunks form one equal-length run
    (fixed-length kernels, decode with its fused write, the tail launch),
    captured in one HIP graph: every replay, from restored caches, reproduces
    the eager outputs, LSE and caches bit for bit."""
    print("first chunk + mixed step graph replay", flush=True)
    B, Hq, Hkv, D, W, S = 4, 8, 2, 128, 100, 2
    gpu = GpuSide(B, Hq, Hkv, D, W, S)
    C = 70
    q0 = rnd((B, C, Hq, D), "q", 0, index=96).to(DEV)
    k0 = rnd((B, C, Hkv, D), "k", 0, index=96).to(DEV)
    v0 = rnd((B, C, Hkv, D), "v", 0, index=96).to(DEV)
    st0 = torch.zeros(B, dtype=torch.int32, device=DEV)
    lens = [1, 40, 40, 1]
    T = sum(lens)
    q1 = rnd((T, Hq, D), "chunk_q", 1, index=96).to(DEV)
    k1 = rnd((T, Hkv, D), "chunk_k", 1, index=96).to(DEV)
    v1 = rnd((T, Hkv, D), "chunk_v", 1, index=96).to(DEV)
    st1 = torch.full((B,), C, dtype=torch.int32, device=DEV)
    kr = torch.empty_like(k0)
    o0 = torch.empty((B, C, Hq, D), dtype=torch.bfloat16, device=DEV)
    l0 = torch.empty((B, Hq, C), dtype=torch.float32, device=DEV)
    o1 = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=DEV)
    l1 = torch.empty((Hq, T), dtype=torch.float32, device=DEV)
    ws = torch.empty(swa.swa_step_varlen_workspace_bytes(gpu.p, lens), dtype=torch.uint8, device=DEV)
    kc0, vc0 = gpu.kc.clone(), gpu.vc.clone()

    def run():
        swa.swa_rope_keys_cache_write(gpu.p, k0, v0, st0, gpu.kc, gpu.vc, kr)
        swa.swa_prefill_attention(gpu.p, q0, kr, v0, None, None, st0, o0, l0)
        swa.swa_step_varlen(gpu.p, q1, k1, v1, gpu.kc, gpu.vc, st1, lens, o1, l1, ws)

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o0, l0, o1, l1, gpu.kc, gpu.vc)]
    gpu.kc.copy_(kc0)
    gpu.vc.copy_(vc0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    names = ("out0", "lse0", "out1", "lse1", "k_cache", "v_cache")
    for rep in range(3):
        gpu.kc.copy_(kc0)
        gpu.vc.copy_(vc0)
        for t in (o0, l0, o1, l1):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((o0, l0, o1, l1, gpu.kc, gpu.vc), eager, names):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep}: {name}"
        _ = (gpu.kc.float().sum() + 1).item()   # eager work between replays


def test_decode_long_window_wrap():
    """A 16384-slot buffer (the window of the 16K full-cache comparison)
    filled to its last slot and wrapping to slot 0, through both decode forms,
    against the oracle."""
    print("decode long window wrap", flush=True)
    B, Hq, Hkv, D, W = 1, 8, 2, 128, 16384
    gpu = GpuSide(B, Hq, Hkv, D, W)
    orc = OracleSide(range(B), Hkv, D, W)
    p0 = W - 6
    kh = rnd((1, p0, Hkv, D), "hist_k", 0, index=95)
    vh = rnd((1, p0, Hkv, D), "hist_v", 0, index=95)
    gpu.write(kh, vh, [0])
    orc.write(kh, vh, [0])
    atol, rrms, latol = tol(torch.bfloat16)
    for st in range(12):   # positions W-6 .. W+5: the fill point, then slots 0..5 overwritten
        q = rnd((B, Hq, D), "step_q", st, index=95)
        k = rnd((B, Hkv, D), "step_k", st, index=95)
        v = rnd((B, Hkv, D), "step_v", st, index=95)
        pos = [p0 + st]
        out, lse = gpu.decode(q, k, v, pos, fused=st % 2 == 1)
        ref = orc.decode(q, k, v, pos)
        assert_close(out[0], ref[0][0], atol, rrms, f"step {st} out")
        assert_lse(lse[0], ref[0][1], latol, f"step {st} lse")
