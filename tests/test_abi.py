"""The C ABI on the CPU: the library loads without a GPU, exports every symbol
include/swa.h declares, and rejects bad arguments on the host before any HIP
call (no kernel is ever launched here)."""
import ctypes
import os
import re

import pytest

import sliding_window_gqa_amd as swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(swa.LIB_PATH),
                                reason="libswa.so not built (run __graft_entry__.build())")

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(swa_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"swa_cache_write", "swa_prefill_chunk", "swa_decode", "swa_decode_step",
            "swa_decode_workspace_bytes",
            "swa_rope_keys", "swa_prefill_attention",
            "swa_prefill_workspace_bytes", "swa_status_string", "swa_debug_slots",
            "swa_debug_mask", "swa_prefill_varlen_workspace_bytes", "swa_rope_keys_varlen",
            "swa_prefill_attention_varlen", "swa_prefill_chunk_varlen",
            "swa_cache_write_varlen", "swa_step_varlen",
            "swa_step_varlen_workspace_bytes", "swa_decode_step_noalloc",
            "swa_noalloc_scratch_bytes", "swa_rope_keys_cache_write",
            "swa_prefill_chunk_aligned", "swa_prefill_chunk_aligned_write_prev"} <= set(names)
    lib = ctypes.CDLL(swa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def P(**kw):
    base = dict(batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128, window=4096, n_sink=0,
                scale=0.0, rope_theta=10000.0, dtype=swa.SWA_BF16)
    base.update(kw)
    return swa.make_params(**base)


BAD_PARAMS = [
    (dict(n_q_heads=30), swa.SWA_ERR_SHAPE),        # Hq % Hkv != 0
    (dict(head_dim=96), swa.SWA_ERR_SHAPE),
    (dict(window=0), swa.SWA_ERR_SHAPE),
    (dict(n_sink=-1), swa.SWA_ERR_SHAPE),
    (dict(n_sink=4097), swa.SWA_ERR_SHAPE),
    (dict(batch=0), swa.SWA_ERR_SHAPE),
    (dict(scale=-1.0), swa.SWA_ERR_SHAPE),
    (dict(scale=float("nan")), swa.SWA_ERR_SHAPE),
    (dict(rope_theta=-5.0), swa.SWA_ERR_SHAPE),
    (dict(dtype=7), swa.SWA_ERR_DTYPE),
]


@pytest.mark.parametrize("bad,code", BAD_PARAMS)
def test_bad_params_rejected_everywhere(bad, code):
    lib = swa.library()
    p = P(**bad)
    bp = ctypes.byref(p)
    assert lib.swa_cache_write(bp, FAKE, FAKE, FAKE, 4, FAKE, FAKE, None) == code
    assert lib.swa_prefill_chunk(bp, FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE, None, FAKE, 1 << 30, None) == code
    assert lib.swa_prefill_chunk_aligned(bp, FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE, None, FAKE, 1 << 30,
                                         None) == code
    assert lib.swa_prefill_chunk_aligned_write_prev(bp, FAKE, FAKE, FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                    16, FAKE, None, FAKE, 1 << 30, None) == code
    assert lib.swa_decode(bp, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == code
    assert lib.swa_decode_step(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == code
    assert lib.swa_decode_step_noalloc(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == code
    assert lib.swa_debug_slots(bp, FAKE, 4, FAKE, None) == code
    assert lib.swa_rope_keys(bp, FAKE, FAKE, 4, FAKE, None) == code
    assert lib.swa_rope_keys_cache_write(bp, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None) == code
    assert lib.swa_prefill_attention(bp, FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE, None, None) == code
    assert lib.swa_decode_workspace_bytes(bp) == 0
    assert lib.swa_prefill_workspace_bytes(bp, 16) == 0


def test_null_pointers_rejected():
    lib = swa.library()
    bp = ctypes.byref(P())
    assert lib.swa_cache_write(None, FAKE, FAKE, FAKE, 4, FAKE, FAKE, None) == swa.SWA_ERR_NULL
    assert lib.swa_cache_write(bp, None, FAKE, FAKE, 4, FAKE, FAKE, None) == swa.SWA_ERR_NULL
    assert lib.swa_cache_write(bp, FAKE, FAKE, None, 4, FAKE, FAKE, None) == swa.SWA_ERR_NULL
    assert lib.swa_cache_write(bp, FAKE, FAKE, FAKE, 4, FAKE, None, None) == swa.SWA_ERR_NULL
    assert lib.swa_prefill_chunk(bp, None, FAKE, FAKE, None, None, FAKE, 16, FAKE, None, FAKE, 1 << 30, None) == swa.SWA_ERR_NULL
    # exactly one cache pointer given
    assert lib.swa_prefill_chunk(bp, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, FAKE, None, FAKE, 1 << 30, None) == swa.SWA_ERR_NULL
    for i in range(5):   # q, k, v, start_pos, out
        args = [FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE]
        args[[0, 1, 2, 5, 7][i]] = None
        assert lib.swa_prefill_chunk_aligned(bp, *args, None, FAKE, 1 << 30, None) == swa.SWA_ERR_NULL, i
    assert lib.swa_prefill_chunk_aligned(bp, FAKE, FAKE, FAKE, None, FAKE, FAKE, 16, FAKE, None, FAKE, 1 << 30,
                                         None) == swa.SWA_ERR_NULL
    for ap in (P(), P(n_sink=4)):   # fused, and the two calls it makes with sinks
        b2 = ctypes.byref(ap)
        for i in range(10):   # k_prev, v_prev, start_prev, q, k, v, k_cache, v_cache, start_pos, out
            args = [FAKE] * 10
            args[i] = None
            assert lib.swa_prefill_chunk_aligned_write_prev(b2, *args[:3], 16, *args[3:9], 16, args[9], None, FAKE,
                                                            1 << 30, None) == swa.SWA_ERR_NULL, i
    assert lib.swa_decode(bp, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 30, None) == swa.SWA_ERR_NULL
    for i in range(7):   # q, k, v, k_cache, v_cache, pos, out
        args = [FAKE] * 7
        args[i] = None
        assert lib.swa_decode_step(bp, *args, None, FAKE, 1 << 30, None) == swa.SWA_ERR_NULL, i
    assert lib.swa_debug_mask(bp, 5, None, 4, FAKE, None) == swa.SWA_ERR_NULL
    assert lib.swa_rope_keys(bp, FAKE, FAKE, 4, None, None) == swa.SWA_ERR_NULL
    for i in range(6):   # k, v, start_pos, k_rot, k_cache, v_cache
        args = [FAKE] * 6
        args[i] = None
        assert lib.swa_rope_keys_cache_write(bp, *args[:3], 4, *args[3:], None) == swa.SWA_ERR_NULL, i
    assert lib.swa_prefill_attention(bp, FAKE, None, FAKE, None, None, FAKE, 16, FAKE, None, None) == swa.SWA_ERR_NULL
    assert lib.swa_prefill_attention(bp, FAKE, FAKE, FAKE, None, FAKE, FAKE, 16, FAKE, None, None) == swa.SWA_ERR_NULL


def test_sizes_and_workspace_rejected():
    lib = swa.library()
    p = P()
    bp = ctypes.byref(p)
    assert lib.swa_cache_write(bp, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None) == swa.SWA_ERR_SHAPE
    assert lib.swa_rope_keys_cache_write(bp, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None) == swa.SWA_ERR_SHAPE
    assert lib.swa_prefill_chunk(bp, FAKE, FAKE, FAKE, None, None, FAKE, 0, FAKE, None, FAKE, 1 << 30, None) == swa.SWA_ERR_SHAPE
    need = lib.swa_prefill_workspace_bytes(bp, 16)
    assert lib.swa_prefill_chunk(bp, FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE, None, FAKE, need - 1, None) == swa.SWA_ERR_WORKSPACE
    assert lib.swa_prefill_chunk(bp, FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE, None, None, need, None) == swa.SWA_ERR_WORKSPACE
    for ap in (P(), P(n_sink=4)):   # the aligned path, and its fallback to swa_prefill_chunk (sinks)
        b2 = ctypes.byref(ap)
        assert lib.swa_prefill_chunk_aligned(b2, FAKE, FAKE, FAKE, None, None, FAKE, 0, FAKE, None, FAKE, 1 << 30,
                                             None) == swa.SWA_ERR_SHAPE
        assert lib.swa_prefill_chunk_aligned(b2, FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE, None, FAKE, need - 1,
                                             None) == swa.SWA_ERR_WORKSPACE
        assert lib.swa_prefill_chunk_aligned(b2, FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE, None, None, need,
                                             None) == swa.SWA_ERR_WORKSPACE
        wp = lib.swa_prefill_chunk_aligned_write_prev
        for plen, clen, ws, w_need in ((0, 16, FAKE, need), (16, 0, FAKE, need), (16, 16, FAKE, need - 1),
                                       (16, 16, None, need)):
            code = swa.SWA_ERR_SHAPE if plen < 1 or clen < 1 else swa.SWA_ERR_WORKSPACE
            assert wp(b2, FAKE, FAKE, FAKE, plen, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, clen, FAKE, None, ws, w_need,
                      None) == code, (plen, clen)
    dneed = lib.swa_decode_workspace_bytes(bp)
    assert lib.swa_decode(bp, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, dneed - 1, None) == swa.SWA_ERR_WORKSPACE
    assert lib.swa_decode_step(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, dneed - 1, None) == swa.SWA_ERR_WORKSPACE
    assert lib.swa_decode_step(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, dneed, None) == swa.SWA_ERR_WORKSPACE
    assert lib.swa_debug_slots(bp, FAKE, 0, FAKE, None) == swa.SWA_ERR_SHAPE
    assert lib.swa_debug_mask(bp, -1, FAKE, 4, FAKE, None) == swa.SWA_ERR_SHAPE


def test_workspace_sizes():
    lib = swa.library()
    # prefill: the chunk's rotated keys, one element per (b, token, kv head, dim)
    for dt, es in ((swa.SWA_BF16, 2), (swa.SWA_F32, 4)):
        p = P(dtype=dt)
        assert lib.swa_prefill_workspace_bytes(ctypes.byref(p), 4096) == 2 * 4096 * 8 * 128 * es
    # decode: B*Hq partials of (D + 2) floats per split; splits cover the slots
    for B, W, S in ((64, 4096, 0), (16, 4092, 4), (1, 64, 0), (3, 100, 2)):
        p = P(batch=B, window=W, n_sink=S)
        nbytes = lib.swa_decode_workspace_bytes(ctypes.byref(p))
        per_split = B * 32 * (128 + 2) * 4
        assert nbytes % per_split == 0
        n_splits = nbytes // per_split
        assert 1 <= n_splits <= -(-(W + S) // 256)
        assert B * 8 * n_splits >= min(256, B * 8 * -(-(W + S) // 256))


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        s = swa.swa_status_string(code)
        assert s.startswith("SWA_")
    assert "unknown" in swa.swa_status_string(42)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(swa, "_lib", None)
    monkeypatch.setattr(swa, "LIB_PATH", str(tmp_path / "libswa.so"))
    with pytest.raises(RuntimeError, match="missing"):
        swa.library()


def _lens(*xs):
    return (ctypes.c_int32 * len(xs))(*xs)


def test_varlen_arguments_rejected():
    lib = swa.library()
    p = P(batch=3)
    bp = ctypes.byref(p)
    good = _lens(5, 0, 7)
    calls = [
        lambda L: lib.swa_rope_keys_varlen(bp, FAKE, FAKE, L, FAKE, None),
        lambda L: lib.swa_cache_write_varlen(bp, FAKE, FAKE, FAKE, L, FAKE, FAKE, None),
        lambda L: lib.swa_prefill_attention_varlen(bp, FAKE, FAKE, FAKE, None, None, FAKE, L, FAKE, None, None),
        lambda L: lib.swa_prefill_chunk_varlen(bp, FAKE, FAKE, FAKE, None, None, FAKE, L, FAKE, None, FAKE,
                                               1 << 30, None),
        lambda L: lib.swa_step_varlen(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, L, FAKE, None, FAKE, 1 << 30, None),
    ]
    for call in calls:
        assert call(None) == swa.SWA_ERR_NULL
        assert call(_lens(0, 0, 0)) == swa.SWA_ERR_SHAPE       # no token at all
        assert call(_lens(5, -1, 7)) == swa.SWA_ERR_SHAPE
        assert call(_lens(5, (1 << 24) + 1, 7)) == swa.SWA_ERR_SHAPE
    # bad params come first, before the lengths are read
    bad = ctypes.byref(P(batch=3, head_dim=96))
    assert lib.swa_rope_keys_varlen(bad, FAKE, FAKE, good, FAKE, None) == swa.SWA_ERR_SHAPE
    assert lib.swa_prefill_varlen_workspace_bytes(bad, good) == 0
    assert lib.swa_prefill_varlen_workspace_bytes(bp, None) == 0
    # workspace: the packed rotated keys
    need = lib.swa_prefill_varlen_workspace_bytes(bp, good)
    assert need == 12 * 8 * 128 * 2
    assert lib.swa_prefill_chunk_varlen(bp, FAKE, FAKE, FAKE, None, None, FAKE, good, FAKE, None, FAKE,
                                        need - 1, None) == swa.SWA_ERR_WORKSPACE
    assert lib.swa_prefill_chunk_varlen(bp, FAKE, FAKE, FAKE, FAKE, None, FAKE, good, FAKE, None, FAKE,
                                        need, None) == swa.SWA_ERR_NULL   # one cache pointer only


def test_step_varlen_workspace():
    lib = swa.library()
    p = P(batch=4)
    bp = ctypes.byref(p)
    # no one-token sequence: the rotated keys only (rounded up to 256 bytes)
    assert lib.swa_step_varlen_workspace_bytes(bp, _lens(5, 3, 0, 9)) == -(-(17 * 8 * 128 * 2) // 256) * 256
    assert lib.swa_step_varlen_workspace_bytes(bp, _lens(5, 3, 0, 2)) == -(-(10 * 8 * 128 * 2) // 256) * 256
    # two one-token sequences: plus their split-K partials
    # (the 30-token chunk is a run of one: its LSE [1][32][30] has room of its own)
    nbytes = lib.swa_step_varlen_workspace_bytes(bp, _lens(1, 30, 1, 0))
    keys = 32 * 8 * 128 * 2
    assert nbytes == keys + 2 * 32 * 16 * 130 * 4 + 1 * 32 * 30 * 4   # 16 splits for 2 x 8 KV heads
    for i in range(3):
        args = [FAKE] * 6    # q, k, v, k_cache, v_cache, start_pos
        args[3 + i] = None
        assert lib.swa_step_varlen(bp, *args, _lens(1, 30, 1, 0), FAKE, None, FAKE, 1 << 30, None) == swa.SWA_ERR_NULL
    assert lib.swa_step_varlen(bp, *([FAKE] * 6), _lens(1, 30, 1, 0), FAKE, None, FAKE, nbytes - 1,
                               None) == swa.SWA_ERR_WORKSPACE


def test_step_varlen_workspace_equal_runs():
    """Chunks of one length in one contiguous run: the step's fixed-length
    path packs the run's LSE ([run][Hq][len] floats) through the workspace;
    chunks of different lengths take the varlen kernel and need no such room."""
    lib = swa.library()
    p = P(batch=4)
    bp = ctypes.byref(p)
    keys = 80 * 8 * 128 * 2
    assert lib.swa_step_varlen_workspace_bytes(bp, _lens(0, 40, 40, 0)) == keys + 2 * 32 * 40 * 4
    assert lib.swa_step_varlen_workspace_bytes(bp, _lens(40, 40, 3, 0)) == -(-(83 * 8 * 128 * 2) // 256) * 256
    assert lib.swa_step_varlen_workspace_bytes(bp, _lens(40, 0, 40, 0)) == keys   # not contiguous


def test_step_varlen_workspace_over_several_decode_launches():
    """70 one-token sequences decode in two launches (64 + 6); the smaller
    launch takes more splits, and the workspace holds the larger need."""
    lib = swa.library()
    p = P(batch=70)

    def splits(b):   # about 256 work-groups, ranges of at least 256 slots
        return max(1, min(-(-256 // (b * 8)), -(-4096 // 256)))

    part = max(b * 32 * splits(b) * 130 * 4 for b in (64, 6))
    keys = -(-(70 * 8 * 128 * 2) // 256) * 256
    assert lib.swa_step_varlen_workspace_bytes(ctypes.byref(p), _lens(*([1] * 70))) == keys + part
    # float32: keys at 4 bytes per element
    p32 = P(batch=3, dtype=swa.SWA_F32)
    assert lib.swa_prefill_varlen_workspace_bytes(ctypes.byref(p32), _lens(5, 0, 7)) == 12 * 8 * 128 * 4


def test_noalloc_decode_rejects_on_the_host():
    """The no-allocation decode step: null pointers, and shapes whose split-K
    partials need more than the fixed scratch array, are rejected before any
    HIP call."""
    lib = swa.library()
    assert lib.swa_noalloc_scratch_bytes() == 4 << 20
    p = P(batch=4)
    bp = ctypes.byref(p)
    assert lib.swa_decode_step_noalloc(bp, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == swa.SWA_ERR_NULL
    assert lib.swa_decode_step_noalloc(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == swa.SWA_ERR_NULL
    # 4096 sequences on the generic path (float32): one split each, but 4096 x 32
    # partials of 130 floats = 68 MB > 4 MiB
    big = P(batch=4096, dtype=swa.SWA_F32)
    assert lib.swa_decode_workspace_bytes(ctypes.byref(big)) > lib.swa_noalloc_scratch_bytes()
    assert lib.swa_decode_step_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                       None) == swa.SWA_ERR_SCRATCH
    assert "scratch" in swa.swa_status_string(swa.SWA_ERR_SCRATCH)
