"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times.  The oracle evaluates sampled query rows / decode steps one
by one (rows are independent), while it follows every cache write exactly.
"""
import numpy as np
import pytest
import torch

import oracle.swa_oracle as so
import sliding_window_gqa_amd as swa
from sliding_window_gqa_amd import synth
from tests.common import assert_close, assert_lse, tol
from tests.gpu_harness import DEV, GpuSide, OracleSide, np64

pytestmark = pytest.mark.gpu


def sample_rows(C, n_random, seed, fixed, per_tile=True):
    """Query rows the oracle evaluates: the fixed ones (tile and window edges),
    n_random more, and one random row of every 64-query tile (every work item
    of the persistent prefill grid is then compared somewhere)."""
    g = np.random.default_rng(seed)
    rows = set(int(r) for r in fixed if 0 <= r < C)
    rows |= set(int(x) for x in g.choice(C, size=min(n_random, C), replace=False))
    if per_tile:
        rows |= set(int(t0 + g.integers(min(64, C - t0))) for t0 in range(0, C, 64))
    return np.array(sorted(rows))


def check_rows(out, lse, ref, rows, dtype, what):
    atol, rrms, latol = tol(dtype)
    assert_close(out[rows.tolist()], ref[0], atol, rrms, what + " out")
    assert_lse(lse[:, rows.tolist()], ref[1], latol, what + " lse")


def test_workload2_prefill_n8192():
    wl = synth.workload(2)
    print(f"workload {wl.name}", flush=True)
    N, Hq, Hkv, D, W = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    q = synth.normal((1, N, Hq, D), 2, "q")
    k = synth.normal((1, N, Hkv, D), 2, "k")
    v = synth.normal((1, N, Hkv, D), 2, "v")
    gpu = GpuSide(1, Hq, Hkv, D, W)
    out, lse = gpu.prefill(q, k, v, [0], use_cache=False)
    torch.cuda.synchronize()
    rows = sample_rows(N, 24, 2, [0, 1, 63, 64, 127, 4095, 4096, 4097, 6000, 8191])
    orc = OracleSide([0], Hkv, D, W)
    ref = orc.prefill(q, k, v, [0], rows=rows)[0]
    check_rows(out[0].cpu(), lse[0].cpu(), ref, rows, torch.bfloat16, "prefill n8192")
    # the cache afterwards holds the last W positions
    pos = np.arange(N - W, N)
    np.testing.assert_array_equal(np64(gpu.vc[0])[pos % W], np64(v[0])[pos])


def test_workload3_chunked_prefill_and_full_causal():
    wl = synth.workload(3)
    print(f"workload {wl.name}", flush=True)
    N, Hq, Hkv, D, W, C = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.chunk
    q = synth.normal((1, N, Hq, D), 3, "q")
    k = synth.normal((1, N, Hkv, D), 3, "k")
    v = synth.normal((1, N, Hkv, D), 3, "v")
    gpu = GpuSide(1, Hq, Hkv, D, W)
    orc = OracleSide([0], Hkv, D, W)
    for c in range(N // C):
        s = c * C
        print(f"  chunk {c}", flush=True)
        # the aligned entry (the loop the benchmark times: chunks of W from 0)
        # on the caches as they stand, then the general one, which also writes
        # the chunk into the caches: byte-identical
        st = torch.tensor([s], dtype=torch.int32, device=DEV)
        oa, la = swa.swa_prefill_chunk_aligned(gpu.p, *(x[:, s:s + C].to(DEV) for x in (q, k, v)),
                                               gpu.kc if c else None, gpu.vc if c else None, st)
        out, lse = gpu.prefill(q[:, s:s + C], k[:, s:s + C], v[:, s:s + C], [s])
        assert torch.equal(oa.view(torch.int16), out.view(torch.int16)), f"chunk {c}: aligned out differs"
        assert torch.equal(la.view(torch.int32), lse.view(torch.int32)), f"chunk {c}: aligned lse differs"
        rows = sample_rows(C, 12, 30 + c, [0, 1, 2, 63, 64, 2047, 4094, 4095])
        ref = orc.prefill(q[:, s:s + C], k[:, s:s + C], v[:, s:s + C], [s], rows=rows)[0]
        check_rows(out[0].cpu(), lse[0].cpu(), ref, rows, torch.bfloat16, f"chunk {c}")
        np.testing.assert_array_equal(np.sort(orc.caches[0].positions()), np.arange(s + C - W, s + C))
    # full causal attention at N = 16384 (window >= N), one pass
    Wf = wl.extra["full_window"]
    print("  full causal", flush=True)
    gfull = GpuSide(1, Hq, Hkv, D, Wf)
    out, lse = gfull.prefill(q, k, v, [0], use_cache=False)
    rows = sample_rows(N, 12, 39, [0, 1, 8191, 16383])
    ref = OracleSide([0], Hkv, D, Wf).prefill(q, k, v, [0], rows=rows)[0]
    check_rows(out[0].cpu(), lse[0].cpu(), ref, rows, torch.bfloat16, "full causal")


def _decode_setup(wl, n_oracle_seqs, seed):
    B, Hq, Hkv, D, W, S = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.n_sink
    p0 = synth.positions(wl.index, B, wl.pos_lo, wl.pos_hi).numpy().astype(np.int64)
    gpu = GpuSide(B, Hq, Hkv, D, W, S)
    # the buffers start out holding N(0,1) values in every slot
    for b in range(B):
        gpu.kc[b] = synth.normal(gpu.kc.shape[1:], wl.index, "garbage_k", b).to(DEV)
        gpu.vc[b] = synth.normal(gpu.vc.shape[1:], wl.index, "garbage_v", b).to(DEV)
    order = np.argsort(p0)
    g = np.random.default_rng(seed)
    seqs = sorted(set(order[:4].tolist()) | set(g.choice(B, size=n_oracle_seqs - 4, replace=False).tolist()))
    orc = OracleSide(seqs, Hkv, D, W, S)
    return p0, gpu, orc


def test_workload4_batched_decode():
    wl = synth.workload(4)
    print(f"workload {wl.name}", flush=True)
    B, Hq, Hkv, D, W = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    p0, gpu, orc = _decode_setup(wl, 16, 4)
    # history: positions max(0, p0-W) .. p0-1 hold N(0,1) keys taken as already rotated
    p_one = swa.make_params(1, Hq, Hkv, D, W, 0, 0.0, 0.0)
    for b in range(B):
        lo = max(0, int(p0[b]) - W)
        n = int(p0[b]) - lo
        if n == 0:
            continue
        kh = synth.normal((1, n, Hkv, D), 4, "hist_k", b)
        vh = synth.normal((1, n, Hkv, D), 4, "hist_v", b)
        swa.swa_cache_write(p_one, kh.to(DEV), vh.to(DEV), torch.tensor([lo], dtype=torch.int32, device=DEV),
                            gpu.kc[b:b + 1], gpu.vc[b:b + 1])
        if b in orc.caches:
            orc.caches[b].write(np64(kh[0]), np64(vh[0]), np.arange(lo, int(p0[b])))
    qs = synth.normal((wl.steps, B, Hq, D), 4, "step_q")
    ks = synth.normal((wl.steps, B, Hkv, D), 4, "step_k")
    vs = synth.normal((wl.steps, B, Hkv, D), 4, "step_v")
    check_at = {0, 1, 2, 127, 254, 255}
    atol, rrms, latol = tol(torch.bfloat16)
    for s in range(wl.steps):
        pos = p0 + s
        out, lse = gpu.decode(qs[s], ks[s], vs[s], pos, fused=True)   # as the benchmark times it
        ref = orc.decode(qs[s], ks[s], vs[s], pos, compute=s in check_at)
        if s in check_at:
            o, l = out.cpu(), lse.cpu()
            for b, (ro, rl) in ref.items():
                assert_close(o[b], ro, atol, rrms, f"step {s} seq {b} (p={pos[b]})")
                assert_lse(l[b], rl, latol, f"step {s} seq {b} lse")


def test_workload5_sink_streaming():
    wl = synth.workload(5)
    print(f"workload {wl.name}", flush=True)
    B, Hq, Hkv, D, W, S = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.n_sink
    p0, gpu, orc = _decode_setup(wl, 8, 5)
    ksk = synth.normal((B, S, Hkv, D), 5, "sink_k")
    vsk = synth.normal((B, S, Hkv, D), 5, "sink_v")
    gpu.write(ksk, vsk, [0] * B)
    orc.write(ksk, vsk, [0] * B)
    kh = synth.normal((B, W, Hkv, D), 5, "hist_k")
    vh = synth.normal((B, W, Hkv, D), 5, "hist_v")
    gpu.write(kh, vh, p0 - W)
    orc.write(kh, vh, p0 - W)
    atol, rrms, latol = tol(torch.bfloat16)
    p = p0.copy()
    for phase in range(2):
        qs = synth.normal((wl.steps, B, Hq, D), 5, "step_q", phase)
        ks = synth.normal((wl.steps, B, Hkv, D), 5, "step_k", phase)
        vs = synth.normal((wl.steps, B, Hkv, D), 5, "step_v", phase)
        for s in range(wl.steps):
            check = s in (0, wl.steps - 1)
            # phase 0: cache write + decode as two calls; phase 1: one swa_decode_step
            out, lse = gpu.decode(qs[s], ks[s], vs[s], p, fused=phase == 1)
            ref = orc.decode(qs[s], ks[s], vs[s], p, compute=check)
            if check:
                o, l = out.cpu(), lse.cpu()
                for b, (ro, rl) in ref.items():
                    assert_close(o[b], ro, atol, rrms, f"phase {phase} step {s} seq {b}")
                    assert_lse(l[b], rl, latol, f"phase {phase} step {s} seq {b} lse")
            p = p + 1
        if phase == 0:
            print("  chunk", flush=True)
            C = wl.chunk
            qc = synth.normal((B, C, Hq, D), 5, "chunk_q")
            kc = synth.normal((B, C, Hkv, D), 5, "chunk_k")
            vc = synth.normal((B, C, Hkv, D), 5, "chunk_v")
            out, lse = gpu.prefill(qc, kc, vc, p)
            o, l = out.cpu(), lse.cpu()
            for i, b in enumerate(orc.seqs):
                # every 64-query tile on half the followed sequences
                rows = sample_rows(C, 6, 55 + b, [0, 1, 4095], per_tile=i % 2 == 0)
                ref = so.prefill_chunk(orc.caches[b], np64(qc[b]), np64(kc[b]), np64(vc[b]), int(p[b]),
                                       orc.theta, orc.scale, rows=rows)
                check_rows(o[b], l[b], ref, rows, torch.bfloat16, f"chunk seq {b}")
            p = p + C


def test_mixed_varlen_step_b64():
    """The mixed batch of the benchmark's context at full size: 64 sequences
    with full 4096-slot windows, 4 of them prefill a 1024-token chunk and 60
    decode one token, in one swa_step_varlen.  The oracle follows 8 sequences
    (the 4 chunks on sampled rows, 4 decodes) through their history and the
    step."""
    wl = synth.workload(4)
    print("mixed varlen step b64", flush=True)
    B, Hq, Hkv, D, W = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    n_pre, chunk = 4, 1024
    lens = [chunk] * n_pre + [1] * (B - n_pre)
    starts = synth.positions(94, B, W, 32768).numpy().astype(np.int64)
    seqs = [0, 1, 2, 3, 4, 17, 40, 63]
    gpu = GpuSide(B, Hq, Hkv, D, W)
    orc = OracleSide(seqs, Hkv, D, W)
    # history: the W positions before each start (N(0,1) keys taken as already rotated)
    p_one = swa.make_params(1, Hq, Hkv, D, W, 0, 0.0, 0.0)
    for b in range(B):
        kh = synth.normal((1, W, Hkv, D), 94, "hist_k", b)
        vh = synth.normal((1, W, Hkv, D), 94, "hist_v", b)
        lo = int(starts[b]) - W
        swa.swa_cache_write(p_one, kh.to(DEV), vh.to(DEV), torch.tensor([lo], dtype=torch.int32, device=DEV),
                            gpu.kc[b:b + 1], gpu.vc[b:b + 1])
        if b in orc.caches:
            orc.caches[b].write(np64(kh[0]), np64(vh[0]), np.arange(lo, int(starts[b])))
    T = sum(lens)
    q = synth.normal((T, Hq, D), 94, "chunk_q")
    k = synth.normal((T, Hkv, D), 94, "chunk_k")
    v = synth.normal((T, Hkv, D), 94, "chunk_v")
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    out, lse = swa.swa_step_varlen(gpu.p, q.to(DEV), k.to(DEV), v.to(DEV), gpu.kc, gpu.vc, st, lens)
    o, l = out.cpu(), lse.cpu()
    rows = sample_rows(chunk, 6, 94, [0, 1, 63, 64, 1023])
    offs = np.concatenate([[0], np.cumsum(lens)])
    for b in seqs:
        r0, n = int(offs[b]), lens[b]
        if n > 1:
            ref = so.prefill_chunk(orc.caches[b], np64(q[r0:r0 + n]), np64(k[r0:r0 + n]), np64(v[r0:r0 + n]),
                                   int(starts[b]), 10000.0, rows=rows)
            check_rows(o[r0:r0 + n], l[:, r0:r0 + n], ref, rows, torch.bfloat16, f"chunk seq {b}")
        else:
            ref = so.prefill_chunk(orc.caches[b], np64(q[r0:r0 + 1]), np64(k[r0:r0 + 1]), np64(v[r0:r0 + 1]),
                                   int(starts[b]), 10000.0)
            check_rows(o[r0:r0 + 1], l[:, r0:r0 + 1], ref, np.array([0]), torch.bfloat16, f"decode seq {b}")
        # the rolling buffer after the step holds the oracle's entries (which
        # now include the step's): values verbatim, keys to bf16 rounding
        c = orc.caches[b]
        held = c.tag >= 0
        kc_b, vc_b = np64(gpu.kc[b]), np64(gpu.vc[b])
        np.testing.assert_array_equal(vc_b[held], c.v[held])
        err = np.abs(kc_b[held] - c.k[held])
        assert (err <= 2.0 ** -8 * np.abs(c.k[held]) + 1e-6).all(), (b, err.max())


def test_rope_keys_cache_write_full_size():
    """The headline layer (8192 tokens, window 4096): the one-pass rotation +
    cache write against swa_rope_keys + swa_cache_write, byte for byte."""
    wl = synth.workload(2)
    print(f"rope_keys_cache_write {wl.name}", flush=True)
    N, Hq, Hkv, D, W = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    p = swa.make_params(1, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta)
    k = synth.normal((1, N, Hkv, D), 2, "k").to(DEV)
    v = synth.normal((1, N, Hkv, D), 2, "v").to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    kc1 = torch.full((1, W, Hkv, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc1 = kc1.clone()
    kc2, vc2 = kc1.clone(), vc1.clone()
    kr1 = swa.swa_rope_keys(p, k, st)
    swa.swa_cache_write(p, k, v, st, kc1, vc1)
    kr2 = swa.swa_rope_keys_cache_write(p, k, v, st, kc2, vc2)
    for a, b, what in ((kr1, kr2, "k_rot"), (kc1, kc2, "k_cache"), (vc1, vc2, "v_cache")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), what
