"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

None of these re-types the oracle's own formula: each compares the oracle
against a library routine, a closed form, a worked example printed on the
pages, an independent brute-force implementation, or an invariant the method
guarantees.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle.swa_oracle as so
from oracle.brute import attend_brute, rope_brute


# Oracle functions are looked up on the module at call time, so that the
# mutation tests can plant a mistake in the oracle and see these pins fail.
def swa_attention(*a, **kw):
    return so.swa_attention(*a, **kw)


def rope(*a, **kw):
    return so.rope(*a, **kw)


def key_mask(*a, **kw):
    return so.key_mask(*a, **kw)


def prefill_chunk(*a, **kw):
    return so.prefill_chunk(*a, **kw)


def decode_step(*a, **kw):
    return so.decode_step(*a, **kw)


def kv_cache_bytes(*a, **kw):
    return so.kv_cache_bytes(*a, **kw)


def RollingCache(*a, **kw):
    return so.RollingCache(*a, **kw)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# W >= N reduces to ordinary causal attention (torch's SDPA, fp64, CPU)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,Hq,Hkv,D", [(37, 4, 1, 16), (64, 8, 2, 32), (50, 4, 4, 8)])
def test_full_window_equals_sdpa(N, Hq, Hkv, D):
    rng = np.random.default_rng(N * 7 + Hq)
    q, k, v = _rand(rng, N, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    pos = np.arange(N)
    out, lse = swa_attention(q, k, v, pos, pos, window=N)
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)                         # [Hq, N, D]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    s = (tq @ tk.transpose(1, 2)) / math.sqrt(D)
    s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Brute-force scalar softmax on tiny inputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,Hq,Hkv,D,W,S", [
    (12, 4, 2, 8, 4, 0), (10, 2, 1, 6, 1, 0), (15, 6, 3, 4, 5, 2), (9, 4, 1, 8, 20, 0),
    (16, 4, 2, 4, 3, 3),
])
def test_matches_brute_force(N, Hq, Hkv, D, W, S):
    rng = np.random.default_rng(N + W * 11 + S)
    q, k, v = _rand(rng, N, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    pos = np.arange(N)
    out, lse = swa_attention(q, k, v, pos, pos, W, n_sink=S)
    bo, bl = attend_brute(q.tolist(), k.tolist(), v.tolist(), W, n_sink=S)
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-12, atol=1e-13)


def test_rope_matches_brute_force():
    rng = np.random.default_rng(5)
    x = _rand(rng, 7, 3, 16)
    pos = np.array([0, 1, 5, 100, 4095, 32768, 65535])
    got = rope(x, pos, 10000.0)
    for t in range(7):
        for h in range(3):
            np.testing.assert_allclose(got[t, h], rope_brute(x[t, h].tolist(), int(pos[t]), 10000.0),
                                       rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------
def test_window_one_returns_own_value():
    rng = np.random.default_rng(1)
    N, Hq, Hkv, D = 20, 4, 2, 8
    q, k, v = _rand(rng, N, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    pos = np.arange(N)
    out, lse = swa_attention(q, k, v, pos, pos, window=1, scale=0.3)
    for h in range(Hq):
        np.testing.assert_array_equal(out[:, h], v[:, h // 2])
        np.testing.assert_allclose(lse[h], 0.3 * np.einsum("nd,nd->n", q[:, h], k[:, h // 2]), rtol=1e-13)


@pytest.mark.parametrize("W,S", [(5, 0), (8, 0), (6, 2), (100, 0)])
def test_constant_keys_give_window_mean(W, S):
    """Identical keys make every score equal, so the output is the plain mean
    of V over the key set: a windowed moving average (via cumulative sums)."""
    rng = np.random.default_rng(W)
    N, Hq, Hkv, D = 40, 2, 1, 4
    q = _rand(rng, N, Hq, D)
    k = np.repeat(_rand(rng, 1, Hkv, D), N, axis=0)
    v = _rand(rng, N, Hkv, D)
    pos = np.arange(N)
    out, _ = swa_attention(q, k, v, pos, pos, W, n_sink=S)
    csum = np.concatenate([np.zeros((1, D)), np.cumsum(v[:, 0], axis=0)])
    for i in range(N):
        lo = max(0, i - W + 1)
        total = csum[i + 1] - csum[lo]
        count = i + 1 - lo
        n_extra = min(S, lo)               # sinks that fell out of the window
        total = total + csum[n_extra] - csum[0]
        count += n_extra
        for h in range(Hq):
            np.testing.assert_allclose(out[i, h], total / count, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("W,S", [(4, 0), (7, 0), (4096, 0), (4092, 4), (10, 3)])
def test_scale_zero_counts_and_mean_position(W, S):
    """scale = 0 makes attention uniform over A(i): exp(lse) = |A(i)| =
    min(i+1, W) (+ sinks outside the window), and with v_j = j the output is the
    mean attended position; for the window part that is (lo + i) / 2."""
    N = 3 * W + 5 if W < 100 else W + 300
    pos = np.arange(N)
    q = np.ones((N, 1, 2))
    k = np.ones((N, 1, 2))
    v = np.repeat(pos.astype(np.float64)[:, None, None], 2, axis=2)
    out, lse = swa_attention(q, k, v, pos, pos, W, n_sink=S, scale=0.0, rows_per_pass=512)
    for i in range(N):
        lo = max(0, i - W + 1)
        n_win = i - lo + 1
        n_extra = min(S, lo)
        count = n_win + n_extra
        assert round(math.exp(lse[0, i])) == count
        assert abs(lse[0, i] - math.log(count)) < 1e-12
        mean = (n_win * (lo + i) / 2 + n_extra * (n_extra - 1) / 2) / count
        assert abs(out[i, 0, 0] - mean) < 1e-9


def test_key_set_of_decode_is_read_range():
    """Digest page, "읽기(read) 단계": the query at p reads positions p-W+1 .. p."""
    W = 6
    for p in range(0, 30):
        got = np.nonzero(key_mask([p], np.arange(40), W)[0])[0]
        np.testing.assert_array_equal(got, np.arange(max(0, p - W + 1), p + 1))


def test_gqa_equals_mha_with_replicated_kv():
    """Explainer, How It Works 1: each subset of query heads shares one K/V head;
    replicating every K/V head over its group (contiguous subsets) and running
    multi-head attention must give the same result."""
    rng = np.random.default_rng(2)
    N, Hq, Hkv, D = 24, 8, 2, 8
    q, k, v = _rand(rng, N, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    pos = np.arange(N)
    out, lse = swa_attention(q, k, v, pos, pos, 5)
    out2, lse2 = swa_attention(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), pos, pos, 5)
    np.testing.assert_allclose(out, out2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-13)
    # and each head group really uses its own K/V head: changing K/V head 1
    # leaves heads 0..3 unchanged and changes heads 4..7
    k2 = k.copy()
    k2[:, 1] = _rand(rng, N, D)
    out3, _ = swa_attention(q, k2, v, pos, pos, 5)
    np.testing.assert_allclose(out3[:, :4], out[:, :4], rtol=1e-13, atol=1e-13)
    assert np.abs(out3[:, 4:] - out[:, 4:]).max() > 1e-3


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def test_rope_closed_form_angles():
    """Unit vector e_{2k} at position p must become (cos a, sin a) in pair k with
    a = p * theta^(-2k/D).  For D = 128, theta = 10000: pair 0 has frequency 1
    and pair 32 has frequency theta^(-1/2) = 0.01, so p = 1 (pair 0) and
    p = 100 (pair 32) both rotate by exactly 1 radian, counter-clockwise."""
    D = 128
    for kk, p in [(0, 1), (32, 100)]:
        x = np.zeros((1, 1, D))
        x[0, 0, 2 * kk] = 1.0
        y = rope(x, [p], 10000.0)[0, 0]
        assert abs(y[2 * kk] - math.cos(1.0)) < 1e-12
        assert abs(y[2 * kk + 1] - math.sin(1.0)) < 1e-12
        rest = np.delete(y, [2 * kk, 2 * kk + 1])
        assert np.abs(rest).max() == 0.0
    # pair 63 (the slowest): frequency theta^(-126/128)
    x = np.zeros((1, 1, D))
    x[0, 0, 127] = 1.0
    y = rope(x, [1000], 10000.0)[0, 0]
    a = 1000 * 10000.0 ** (-126 / 128)
    assert abs(y[126] + math.sin(a)) < 1e-12 and abs(y[127] - math.cos(a)) < 1e-12


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(3)
    x = _rand(rng, 5, 2, 16)
    np.testing.assert_array_equal(rope(x, np.zeros(5, int), 10000.0), x)
    y = rope(x, np.arange(5) * 977, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # scores depend only on i - j: shifting every position leaves attention unchanged
    N, Hq, Hkv, D = 30, 4, 2, 16
    q, k, v = _rand(rng, N, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    pos = np.arange(N)
    o1, l1 = swa_attention(rope(q, pos, 1e4), rope(k, pos, 1e4), v, pos, pos, 7)
    o2, l2 = swa_attention(rope(q, pos + 12345, 1e4), rope(k, pos + 12345, 1e4), v, pos, pos, 7)
    np.testing.assert_allclose(o1, o2, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(l1, l2, rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------------------
# Rolling buffer: the pages' worked example and invariants
# ---------------------------------------------------------------------------
def test_rolling_buffer_w4_worked_example():
    rows = _golden_rows("rolling_buffer_w4.txt")
    cache = RollingCache(1, 2, window=4)
    for r in rows:
        i, slot = int(r[0]), int(r[1])
        held = [int(x) for x in r[2:6]]
        assert cache.slot(i) == slot
        cache.write(np.full((1, 1, 2), float(i)), np.full((1, 1, 2), float(i)), [i])
        assert cache.tag.tolist() == held
        assert cache.v[slot, 0, 0] == float(i)


def test_kv_memory_saving_at_32k():
    (n, w, factor), = [tuple(int(x) for x in r) for r in _golden_rows("kv_memory_32k.txt")]
    shape = {r[0]: int(r[1]) for r in _golden_rows("mistral7b_attention_shape.txt")}
    full = kv_cache_bytes(n, shape["n_layers"], shape["n_kv_heads"], shape["head_dim"], 2)
    cache = RollingCache(1, 1, window=w)
    for p in range(n):                      # write a 32K-token stream
        if p % 97 == 0 or p > n - 3 * w:
            cache.write(np.zeros((1, 1, 1)), np.zeros((1, 1, 1)), [p])
    kept = cache.n_slots
    rolled = kv_cache_bytes(kept, shape["n_layers"], shape["n_kv_heads"], shape["head_dim"], 2)
    assert kept == w
    assert full / rolled == factor
    np.testing.assert_array_equal(cache.positions(), np.arange(n - w, n))


@pytest.mark.parametrize("W,S", [(5, 0), (12, 4), (4092, 4)])
def test_slot_map_is_bijective_on_live_window(W, S):
    cache = RollingCache(1, 1, window=W, n_sink=S)
    for p in list(range(0, 3 * W + 7, max(1, W // 50))) + [3 * W + 7]:
        live = np.nonzero(key_mask([p], np.arange(p + 1), W, S)[0])[0]
        slots = [cache.slot(j) for j in live]
        assert len(set(slots)) == len(slots)
        assert all(0 <= s < W + S for s in slots)
        assert all(cache.slot(j) < S for j in live if j < S)


def test_window_is_at_most_two_contiguous_runs():
    """Digest "읽기(read) 단계": physical slots (p-W+1)%W .. p%W form at most two
    contiguous runs (wrap-around)."""
    W = 16
    cache = RollingCache(1, 1, window=W)
    for p in range(0, 5 * W):
        slots = [cache.slot(j) for j in range(max(0, p - W + 1), p + 1)]
        breaks = sum(1 for a, b in zip(slots, slots[1:]) if b != a + 1)
        assert breaks <= 1


# ---------------------------------------------------------------------------
# Schedules: chunked prefill and decode against the rolling buffer
# ---------------------------------------------------------------------------
def _sequence(rng, N, Hq, Hkv, D):
    return _rand(rng, N, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)


@pytest.mark.parametrize("C", [16, 8, 1, 3, 7, 40])
@pytest.mark.parametrize("S", [0, 2])
def test_chunked_prefill_equals_unchunked(C, S):
    """Essay §4.1 / Figure 3 and explainer How It Works 4: cutting the prompt
    into chunks that attend to the cache plus themselves gives the same result
    as one pass, and after each chunk the cache holds the last W positions
    (digest "Pre-fill과의 상호작용")."""
    W, N, Hq, Hkv, D, theta = 16, 61, 4, 2, 8, 10000.0
    rng = np.random.default_rng(C * 3 + S)
    q, k, v = _sequence(rng, N, Hq, Hkv, D)
    pos = np.arange(N)
    ref, ref_lse = swa_attention(rope(q, pos, theta), rope(k, pos, theta), v, pos, pos, W, n_sink=S)
    cache = RollingCache(Hkv, D, W, n_sink=S)
    outs, lses = [], []
    for s in range(0, N, C):
        e = min(N, s + C)
        o, l = prefill_chunk(cache, q[s:e], k[s:e], v[s:e], s, theta)
        outs.append(o)
        lses.append(l)
        expect = sorted(set(range(max(0, e - W), e)) | set(range(min(S, e))))
        np.testing.assert_array_equal(cache.positions(), expect)
    np.testing.assert_allclose(np.concatenate(outs), ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(lses, axis=1), ref_lse, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("S", [0, 3])
def test_rolling_decode_reproduces_full_sequence(S):
    """Decoding tokens 0..N-1 one at a time through the W-slot buffer gives the
    rows of full-sequence SWA (digest "Rolling Buffer KV Cache 동작 설명": the
    buffer keeps everything a query can read)."""
    W, N, Hq, Hkv, D, theta = 8, 45, 4, 1, 8, 10000.0
    rng = np.random.default_rng(10 + S)
    q, k, v = _sequence(rng, N, Hq, Hkv, D)
    pos = np.arange(N)
    ref, ref_lse = swa_attention(rope(q, pos, theta), rope(k, pos, theta), v, pos, pos, W, n_sink=S)
    cache = RollingCache(Hkv, D, W, n_sink=S)
    for p in range(N):
        o, l = decode_step(cache, q[p], k[p], v[p], p, theta)
        np.testing.assert_allclose(o, ref[p], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(l, ref_lse[:, p], rtol=1e-11, atol=1e-12)
        assert len(cache.positions()) == min(p + 1, W + S)


def test_prefill_then_decode_share_one_cache_convention():
    """Digest "Pre-fill과의 상호작용": decode continues from the state the
    prefill left, so prefill of 0..P-1 followed by decode of P..N-1 equals the
    full-sequence rows."""
    W, N, P, Hq, Hkv, D, theta = 10, 40, 23, 4, 2, 8, 10000.0
    rng = np.random.default_rng(77)
    q, k, v = _sequence(rng, N, Hq, Hkv, D)
    pos = np.arange(N)
    ref, _ = swa_attention(rope(q, pos, theta), rope(k, pos, theta), v, pos, pos, W)
    cache = RollingCache(Hkv, D, W)
    o, _ = prefill_chunk(cache, q[:P], k[:P], v[:P], 0, theta)
    np.testing.assert_allclose(o, ref[:P], rtol=1e-11, atol=1e-12)
    for p in range(P, N):
        o, _ = decode_step(cache, q[p], k[p], v[p], p, theta)
        np.testing.assert_allclose(o, ref[p], rtol=1e-11, atol=1e-12)


def test_decode_is_invariant_under_slot_permutation():
    """Softmax is over a set: the slot order of the buffer cannot matter."""
    W, Hq, Hkv, D = 12, 4, 2, 8
    rng = np.random.default_rng(9)
    cache = RollingCache(Hkv, D, W)
    for p in range(30):
        cache.write(_rand(rng, 1, Hkv, D), _rand(rng, 1, Hkv, D), [p])
    q = _rand(rng, 1, Hq, D)
    ck, cv, cpos = cache.entries()
    o1, _ = swa_attention(q, ck, cv, [30 - 1], cpos, W)
    perm = rng.permutation(len(cpos))
    o2, _ = swa_attention(q, ck[perm], cv[perm], [30 - 1], cpos[perm], W)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)


def test_kv_cache_bytes_absolute():
    """The byte count itself, not only the 32K / 4096 ratio: K and V buffers of
    shape (W, n_kv_heads, head_dim) per layer (digest "핵심 구성요소"), bf16,
    32 layers (the architecture table of the digest's "Methods").  Measured
    against the bytes of a real RollingCache's two arrays, rescaled from
    float64 to a 2-byte element, and against the product written out."""
    shape = {r[0]: int(r[1]) for r in _golden_rows("mistral7b_attention_shape.txt")}
    W, L, H, D = 4096, shape["n_layers"], shape["n_kv_heads"], shape["head_dim"]
    cache = RollingCache(H, D, window=W)
    per_layer = (cache.k.nbytes + cache.v.nbytes) // cache.k.itemsize * 2
    assert kv_cache_bytes(W, 1, H, D, 2) == per_layer
    assert kv_cache_bytes(W, L, H, D, 2) == L * per_layer == 536_870_912


# ---------------------------------------------------------------------------
# Dilation (the dilated sliding window the digest lists for Longformer): the
# window part keeps the keys i, i-d, i-2d, ... inside i - W < j <= i
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,Hq,Hkv,D,W,S,d", [
    (14, 4, 2, 4, 9, 0, 2), (17, 2, 1, 6, 12, 2, 3), (11, 4, 1, 4, 5, 1, 5), (13, 4, 2, 4, 20, 0, 4),
    (9, 2, 1, 4, 4, 0, 1),
])
def test_dilated_matches_brute_force(N, Hq, Hkv, D, W, S, d):
    rng = np.random.default_rng(N * 13 + W + 7 * d)
    q, k, v = _rand(rng, N, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    pos = np.arange(N)
    out, lse = swa_attention(q, k, v, pos, pos, W, n_sink=S, dilation=d)
    bo, bl = attend_brute(q.tolist(), k.tolist(), v.tolist(), W, n_sink=S, dilation=d)
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("W,S,d", [(12, 0, 3), (10, 0, 4), (4096, 0, 2), (4092, 4, 3), (9, 5, 2), (7, 0, 1)])
def test_dilated_scale_zero_counts_and_mean_position(W, S, d):
    """scale = 0: exp(lse) counts the keys.  The window part is the progression
    i, i-d, ..., with n = min(ceil(W/d), floor(i/d) + 1) terms and mean
    i - d(n-1)/2; the sinks add the positions below min(S, i+1) that the
    progression does not hit (those of its terms that are below S)."""
    N = 3 * W + 5 if W < 100 else W + 300
    pos = np.arange(N)
    q = np.ones((N, 1, 2))
    k = np.ones((N, 1, 2))
    v = np.repeat(pos.astype(np.float64)[:, None, None], 2, axis=2)
    out, lse = swa_attention(q, k, v, pos, pos, W, n_sink=S, scale=0.0, rows_per_pass=512, dilation=d)
    for i in range(N):
        n = min(-(-W // d), i // d + 1)
        win_sum = n * i - d * n * (n - 1) // 2
        # progression terms below S: k with i - k d < S, i.e. k >= floor((i - S) / d) + 1
        k_lo = 0 if i < S else min(n, (i - S) // d + 1)
        n_low = n - k_lo
        low_sum = sum(i - kk * d for kk in range(k_lo, n))     # (at most S terms)
        m = min(S, i + 1)
        n_extra = m - n_low
        extra_sum = m * (m - 1) // 2 - low_sum
        count = n + n_extra
        assert round(math.exp(lse[0, i])) == count, (i, count)
        assert abs(lse[0, i] - math.log(count)) < 1e-12
        assert abs(out[i, 0, 0] - (win_sum + extra_sum) / count) < 1e-9


@pytest.mark.parametrize("d", [2, 3, 5])
def test_dilation_is_swa_within_each_residue(d):
    """Without sinks, dilated attention never mixes positions of different
    residues mod d: its rows of residue r equal plain SWA (same W, absolute
    positions) over the positions of residue r alone."""
    W, N, Hq, Hkv, D = 11, 47, 4, 2, 8
    rng = np.random.default_rng(100 + d)
    q, k, v = _rand(rng, N, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    pos = np.arange(N)
    out, lse = swa_attention(q, k, v, pos, pos, W, dilation=d)
    for r in range(d):
        sub = pos[pos % d == r]
        o_r, l_r = swa_attention(q[sub], k[sub], v[sub], sub, sub, W)
        np.testing.assert_allclose(out[sub], o_r, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, sub], l_r, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("S,d", [(0, 3), (2, 2), (3, 4)])
def test_dilated_rolling_decode_reproduces_full_sequence(S, d):
    """With W the span in positions, the W-slot rolling buffer holds every key
    of a dilated query: rolling decode of 0..N-1 gives the full-sequence rows."""
    W, N, Hq, Hkv, D, theta = 9, 40, 4, 1, 8, 10000.0
    rng = np.random.default_rng(20 + S + 10 * d)
    q, k, v = _sequence(rng, N, Hq, Hkv, D)
    pos = np.arange(N)
    ref, ref_lse = swa_attention(rope(q, pos, theta), rope(k, pos, theta), v, pos, pos, W, n_sink=S, dilation=d)
    cache = RollingCache(Hkv, D, W, n_sink=S, dilation=d)
    for p in range(N):
        o, l = decode_step(cache, q[p], k[p], v[p], p, theta)
        np.testing.assert_allclose(o, ref[p], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(l, ref_lse[:, p], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("C,d", [(16, 2), (5, 3), (1, 2)])
def test_dilated_chunked_prefill_equals_unchunked(C, d):
    W, N, Hq, Hkv, D, theta, S = 14, 53, 4, 2, 8, 10000.0, 2
    rng = np.random.default_rng(C * 5 + d)
    q, k, v = _sequence(rng, N, Hq, Hkv, D)
    pos = np.arange(N)
    ref, ref_lse = swa_attention(rope(q, pos, theta), rope(k, pos, theta), v, pos, pos, W, n_sink=S, dilation=d)
    cache = RollingCache(Hkv, D, W, n_sink=S, dilation=d)
    outs, lses = [], []
    for s in range(0, N, C):
        e = min(N, s + C)
        o, l = prefill_chunk(cache, q[s:e], k[s:e], v[s:e], s, theta)
        outs.append(o)
        lses.append(l)
    np.testing.assert_allclose(np.concatenate(outs), ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(lses, axis=1), ref_lse, rtol=1e-11, atol=1e-12)
