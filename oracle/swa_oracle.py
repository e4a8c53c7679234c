"""fp64 CPU oracle for causal sliding-window attention with grouped-query heads,
a rolling-buffer KV cache, chunked prefill and single-token decode.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
definition that the HIP library is checked against.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
library never does, and this module imports nothing from the library.

Everything is float64 NumPy, written as the plain definition of what the pages
say the method computes.  Where the pages leave a step open, the reading taken
is stated at that function.  Sources (page title, then the section):

* "Mistral 7B — 슬라이딩 윈도우 어텐션 중심 정리" (blog digest): "Methods"
  (architecture parameters: 32 query / 8 KV heads, head_dim 128, W = 4096,
  RoPE theta = 10000; SWA; rolling buffer; pre-fill + chunking),
  "핵심 구성요소" (the SWA mask, the buffer shape (W, n_kv_heads, head_dim)),
  "Rolling Buffer KV Cache 동작 설명" (write at slot p mod W; the read range of
  a query at p; after each chunk the buffer holds the last W entries).
* "[arXiv 2310.06825] Mistral 7B: 슬라이딩 윈도우 어텐션과 효율 중심 설계로
  재정의한 7B 오픈 LLM" (essay): §2.2 (GQA, SWA), §3.3 (rolling buffer),
  §4.1 and Figure 3 (chunk attends causally to itself and to the window of
  the cache).
* "Mistral 7B: Engineering Extreme Efficiency in LLMs" (explainer): How It
  Works 1 (GQA: query heads grouped into subsets sharing one K/V head),
  2 (the SWA attention equation), 3 (rolling buffer, i mod W), 4 (pre-fill and
  chunking).
* "LLM 추론용 SWA는 ... 캐시를 무한히 키우지 않는 기술에 가깝다" (aionda blog):
  "왜 단순 sliding window만으로는 부족한가" (keep the first few tokens as
  attention sinks next to the recent window).

Readings of the pages (each is also listed in the design notes):

* Window: query at position i attends key j iff j <= i and i - W < j, i.e. W
  keys including itself.  The pages give three versions of the bound; this is
  the one that fits a W-slot buffer written before it is read.
* Sinks: with n_sink > 0 the key set also contains every j < n_sink (j <= i).
  Sink positions keep fixed slots 0..n_sink-1; later positions roll over the
  remaining W slots.
* GQA: query head h uses KV head h // (Hq / Hkv) (contiguous groups).
* RoPE: pairs (2k, 2k+1) rotated by angle p * theta^(-2k/D), counter-clockwise
  (the pair read as a complex number is multiplied by exp(+i*angle)).  Applied
  to queries at their position and to keys at their original position.
* Softmax scale: 1/sqrt(D) unless given.
* Chunked prefill: the chunk's queries attend to the cache as it stood before
  the chunk plus the chunk itself (causal); the chunk is written afterwards.
* Dilation (the digest names Longformer's dilated sliding window as the
  hybrid to try next: "Longformer vs Mistral SWA — 구조적 비교", Open
  Questions (ii), "Discussion"; no page defines it): with dilation d >= 1 the
  window part keeps only the keys j with i - W < j <= i and (i - j) divisible
  by d, i.e. i, i-d, i-2d, ...: ceil(W/d) keys once the history is long
  enough.  W stays the span in positions, so the W-slot rolling buffer still
  holds every key a query can read; Longformer's "w keys with gaps d" is the
  case W = w*d.  Sinks are unaffected.  d = 1 is plain SWA.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "rope",
    "key_mask",
    "swa_attention",
    "RollingCache",
    "prefill_chunk",
    "decode_step",
    "kv_cache_bytes",
]


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def rope(x, pos, theta):
    """Rotary position encoding of ``x`` [T, H, D] at integer positions ``pos`` [T].

    Pair k (elements 2k, 2k+1) is rotated by angle a = p * theta^(-2k/D):
        (x0, x1) -> (x0 cos a - x1 sin a,  x0 sin a + x1 cos a).
    theta = 10000 is the value in the architecture table ("Methods" of the
    digest page).  ``theta == 0`` means no rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    if theta == 0:
        return x.copy()
    T, H, D = x.shape
    pos = np.asarray(pos, dtype=np.float64).reshape(T)
    k = np.arange(D // 2, dtype=np.float64)
    freq = float(theta) ** (-2.0 * k / D)          # [D/2]
    ang = pos[:, None] * freq[None, :]             # [T, D/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ---------------------------------------------------------------------------
# The key set A(i)
# ---------------------------------------------------------------------------
def key_mask(qpos, kpos, window, n_sink=0, dilation=1):
    """Boolean [Tq, Tk]: key at position kpos[j] is in the key set of the query
    at qpos[i].

    SWA mask of the digest page ("핵심 구성요소") and the explainer's SWA
    equation, read as  i - W < j <= i  (W keys including the query itself),
    joined with the sink prefix j < n_sink of the aionda page.  Keys with a
    negative position (an empty cache slot) are never in the set.  With
    dilation d the window part keeps only the keys whose distance i - j is a
    multiple of d (the dilated sliding window the digest lists for
    Longformer; reading in the module header).
    """
    qi = np.asarray(qpos, dtype=np.int64)[:, None]
    kj = np.asarray(kpos, dtype=np.int64)[None, :]
    causal = (kj <= qi) & (kj >= 0)
    in_window = (kj > qi - int(window)) & ((qi - kj) % int(dilation) == 0)
    is_sink = kj < int(n_sink)
    return causal & (in_window | is_sink)


# ---------------------------------------------------------------------------
# Attention over an explicit set of keys
# ---------------------------------------------------------------------------
def swa_attention(q, k, v, qpos, kpos, window, n_sink=0, scale=None, rows_per_pass=256, dilation=1):
    """Sliding-window GQA attention, by definition.

    q [Tq, Hq, D], k and v [Tk, Hkv, D] (already rotated if RoPE is used),
    qpos [Tq], kpos [Tk] absolute positions; A(i) is key_mask's set (with
    ``dilation``).  Returns (out [Tq, Hq, D], lse [Hq, Tq]) where, for query
    head h and KV head g = h // (Hq/Hkv),
        s_ij = scale * q_i . k_j          for j in A(i)
        o_i  = sum_j softmax_j(s_i) v_j   (two-pass: subtract the row max)
        lse_i = log sum_j exp(s_ij)       (natural log)
    Query rows are independent, so they are evaluated ``rows_per_pass`` at a
    time only to bound memory; the arithmetic per row is unchanged.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Hq, D = q.shape
    Tk, Hkv, Dk = k.shape
    assert Dk == D and v.shape == k.shape and Hq % Hkv == 0
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    out = np.empty((Tq, Hq, D), dtype=np.float64)
    lse = np.empty((Hq, Tq), dtype=np.float64)
    for r0 in range(0, Tq, rows_per_pass):
        r1 = min(Tq, r0 + rows_per_pass)
        mask = key_mask(qpos[r0:r1], kpos, window, n_sink, dilation)
        if not mask.any(axis=1).all():
            raise ValueError("a query has an empty key set")
        for h in range(Hq):
            g = h // G
            s = scale * (q[r0:r1, h, :] @ k[:, g, :].T)
            s = np.where(mask, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            out[r0:r1, h, :] = (e @ v[:, g, :]) / l
            lse[h, r0:r1] = m[:, 0] + np.log(l[:, 0])
    return out, lse


# ---------------------------------------------------------------------------
# Rolling-buffer KV cache
# ---------------------------------------------------------------------------
class RollingCache:
    """One sequence's rolling-buffer KV cache for one layer.

    Shape (n_sink + W, n_kv_heads, head_dim), as the digest page gives it
    ("핵심 구성요소": (W, n_kv_heads, head_dim)).  Position p is written to
    slot p mod W (digest "쓰기(write) 단계"; explainer How It Works 3); with
    sinks, positions below n_sink keep slots 0..n_sink-1 and the others roll
    over slots n_sink..n_sink+W-1.

    Every slot carries the position it holds (-1 = empty).  Reads select slots
    by that tag, never by inverting the slot map.
    """

    def __init__(self, n_kv_heads, head_dim, window, n_sink=0, dilation=1):
        self.window = int(window)
        self.n_sink = int(n_sink)
        # the key set the sequence's queries use (the slots do not depend on it)
        self.dilation = int(dilation)
        S = self.n_sink + self.window
        self.k = np.zeros((S, n_kv_heads, head_dim), dtype=np.float64)
        self.v = np.zeros((S, n_kv_heads, head_dim), dtype=np.float64)
        self.tag = np.full(S, -1, dtype=np.int64)

    @property
    def n_slots(self):
        return self.n_sink + self.window

    def slot(self, p):
        p = int(p)
        if p < self.n_sink:
            return p
        return self.n_sink + (p - self.n_sink) % self.window

    def write(self, k_rot, v, positions):
        """Store k_rot[t], v[t] at slot(positions[t]), in order, so a later
        position that lands on the same slot overwrites an earlier one."""
        for t, p in enumerate(np.asarray(positions, dtype=np.int64)):
            s = self.slot(p)
            self.k[s] = k_rot[t]
            self.v[s] = v[t]
            self.tag[s] = int(p)

    def entries(self, below=None):
        """(k, v, positions) of the filled slots, optionally only those holding
        a position < ``below``."""
        sel = self.tag >= 0
        if below is not None:
            sel &= self.tag < int(below)
        return self.k[sel], self.v[sel], self.tag[sel]

    def positions(self):
        return np.sort(self.tag[self.tag >= 0])


def kv_cache_bytes(n_positions_kept, n_layers, n_kv_heads, head_dim, bytes_per_elem):
    """Bytes of a K and V cache holding ``n_positions_kept`` positions."""
    return 2 * n_positions_kept * n_layers * n_kv_heads * head_dim * bytes_per_elem


# ---------------------------------------------------------------------------
# Schedules: one prefill chunk, one decode step
# ---------------------------------------------------------------------------
def prefill_chunk(cache, q, k, v, start, theta=10000.0, scale=None, rows=None):
    """One chunk of chunked prefill for one sequence.

    q [C, Hq, D], k and v [C, Hkv, D] are the raw (un-rotated) projections of
    positions start .. start+C-1.  The chunk's queries attend to the cache
    entries written before the chunk plus the chunk's own keys, within A(i)
    (essay §4.1 and Figure 3; explainer How It Works 4).  The chunk is written
    to the cache afterwards, so after the call the cache holds the last W
    positions (digest "Pre-fill과의 상호작용").  Returns (out, lse).

    ``rows`` (chunk-relative indices) restricts the attention to those query
    rows; every query row is independent, so each returned row is the same as
    in the full evaluation.
    """
    C = q.shape[0]
    pos = np.arange(start, start + C, dtype=np.int64)
    k_rot = rope(k, pos, theta)
    ck, cv, cpos = cache.entries(below=start)
    keys = np.concatenate([ck, k_rot], axis=0)
    vals = np.concatenate([cv, np.asarray(v, dtype=np.float64)], axis=0)
    kpos = np.concatenate([cpos, pos])
    sel = np.arange(C) if rows is None else np.asarray(rows, dtype=np.int64)
    q_rot = rope(np.asarray(q)[sel], pos[sel], theta)
    out, lse = swa_attention(q_rot, keys, vals, pos[sel], kpos, cache.window, cache.n_sink, scale,
                             dilation=cache.dilation)
    cache.write(k_rot, np.asarray(v, dtype=np.float64), pos)
    return out, lse


def decode_step(cache, q, k, v, p, theta=10000.0, scale=None):
    """One decode step for one sequence at position p.

    q [Hq, D], k and v [Hkv, D] raw.  Writes (rope(k, p), v) to slot(p) first
    (digest "쓰기(write) 단계"), then attends q over the cached entries in A(p)
    (digest "읽기(read) 단계").  Returns (out [Hq, D], lse [Hq]).
    """
    pos = np.array([p], dtype=np.int64)
    k_rot = rope(np.asarray(k)[None], pos, theta)
    cache.write(k_rot, np.asarray(v, dtype=np.float64)[None], pos)
    q_rot = rope(np.asarray(q)[None], pos, theta)
    ck, cv, cpos = cache.entries()
    out, lse = swa_attention(q_rot, ck, cv, pos, cpos, cache.window, cache.n_sink, scale,
                             dilation=cache.dilation)
    return out[0], lse[:, 0]
