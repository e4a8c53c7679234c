"""Python binding of libswa: sliding-window GQA attention for MI355X (gfx950).

Thin ctypes layer over the C ABI declared in include/swa.h.  Every function
here has the C name and only marshals arguments (torch tensors -> device
pointers, the current torch stream -> hipStream_t); all arithmetic runs in the
HIP kernels.  The library must have been built (``__graft_entry__.build()`` or
``python -m sliding_window_gqa_amd.build``); a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SwaError", "swa_params", "make_params", "library", "LIB_PATH",
    "swa_cache_write", "swa_prefill_chunk", "swa_prefill_chunk_aligned", "swa_prefill_workspace_bytes",
    "swa_prefill_chunk_aligned_write_prev",
    "swa_decode", "swa_decode_step", "swa_decode_workspace_bytes", "swa_status_string",
    "swa_rope_keys", "swa_prefill_attention", "swa_rope_keys_cache_write",
    "swa_prefill_varlen_workspace_bytes", "swa_rope_keys_varlen", "swa_prefill_attention_varlen",
    "swa_prefill_chunk_varlen", "swa_cache_write_varlen", "swa_step_varlen",
    "swa_step_varlen_workspace_bytes",
    "swa_debug_slots", "swa_debug_mask", "swa_decode_step_noalloc", "swa_noalloc_scratch_bytes",
    "SWA_OK", "SWA_ERR_NULL", "SWA_ERR_SHAPE", "SWA_ERR_DTYPE", "SWA_ERR_UNSUPPORTED",
    "SWA_ERR_WORKSPACE", "SWA_ERR_LAUNCH", "SWA_ERR_SCRATCH", "SWA_BF16", "SWA_F32",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswa.so")

SWA_OK, SWA_ERR_NULL, SWA_ERR_SHAPE, SWA_ERR_DTYPE = 0, -1, -2, -3
SWA_ERR_UNSUPPORTED, SWA_ERR_WORKSPACE, SWA_ERR_LAUNCH, SWA_ERR_SCRATCH = -4, -5, -6, -7
SWA_BF16, SWA_F32 = 0, 1


class SwaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {swa_status_string(status)} ({status})")


class swa_params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("n_sink", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("rope_theta", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("dilation", ctypes.c_int32),
    ]


_P = ctypes.POINTER(swa_params)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

_SIGNATURES = {
    "swa_cache_write": (ctypes.c_int, [_P, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "swa_prefill_workspace_bytes": (_sz, [_P, _i32]),
    "swa_prefill_chunk": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "swa_prefill_chunk_aligned": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "swa_prefill_chunk_aligned_write_prev": (ctypes.c_int, [_P, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp,
                                                            _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "swa_rope_keys": (ctypes.c_int, [_P, _vp, _vp, _i32, _vp, _vp]),
    "swa_rope_keys_cache_write": (ctypes.c_int, [_P, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp]),
    "swa_prefill_attention": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "swa_decode_workspace_bytes": (_sz, [_P]),
    "swa_decode": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "swa_decode_step": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "swa_prefill_varlen_workspace_bytes": (_sz, [_P, _vp]),
    "swa_rope_keys_varlen": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp]),
    "swa_prefill_attention_varlen": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "swa_prefill_chunk_varlen": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "swa_cache_write_varlen": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "swa_step_varlen_workspace_bytes": (_sz, [_P, _vp]),
    "swa_step_varlen": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "swa_decode_step_noalloc": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "swa_noalloc_scratch_bytes": (_sz, []),
    "swa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "swa_debug_slots": (ctypes.c_int, [_P, _vp, _i32, _vp, _vp]),
    "swa_debug_mask": (ctypes.c_int, [_P, _i32, _vp, _i32, _vp, _vp]),
}

_lib = None


def library():
    """Load libswa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sliding_window_gqa_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def swa_status_string(status: int) -> str:
    return library().swa_status_string(int(status)).decode()


def make_params(batch, n_q_heads, n_kv_heads, head_dim, window, n_sink=0, scale=0.0,
                rope_theta=10000.0, dtype=SWA_BF16, dilation=1) -> swa_params:
    if not isinstance(dtype, int):
        import torch
        dtype = SWA_F32 if dtype == torch.float32 else SWA_BF16
    return swa_params(int(batch), int(n_q_heads), int(n_kv_heads), int(head_dim), int(window),
                      int(n_sink), float(scale), float(rope_theta), int(dtype), int(dilation))


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_of(p: swa_params):
    torch = _torch()
    return torch.float32 if p.dtype == SWA_F32 else torch.bfloat16


def _ptr(t, name, dtype=None, shape=None):
    """Device pointer of a contiguous CUDA tensor, after checking it."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status, where):
    if status != SWA_OK:
        raise SwaError(status, where)


def swa_cache_write(params, k, v, start_pos, k_cache, v_cache, stream=None):
    """RoPE the keys and write the tokens k, v [B][n_tok][Hkv][D] at positions
    start_pos[b] + t into the rolling-buffer caches (in place)."""
    torch = _torch()
    dt = _dtype_of(params)
    B, n_tok = k.shape[0], k.shape[1]
    shp = (params.batch, n_tok, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    st = library().swa_cache_write(
        ctypes.byref(params), _ptr(k, "k", dt, shp), _ptr(v, "v", dt, shp),
        _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), n_tok,
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp), _stream(stream))
    _check(st, "swa_cache_write")


def swa_prefill_workspace_bytes(params, chunk_len) -> int:
    return int(library().swa_prefill_workspace_bytes(ctypes.byref(params), int(chunk_len)))


def swa_decode_workspace_bytes(params) -> int:
    return int(library().swa_decode_workspace_bytes(ctypes.byref(params)))


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if workspace is None:
        workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)
    return workspace


def swa_prefill_chunk(params, q, k, v, k_cache, v_cache, start_pos, out=None, lse=None,
                      workspace=None, want_lse=True, stream=None, _entry="swa_prefill_chunk"):
    """Attention of one prefill chunk; returns (out, lse).  Does not write the
    cache (call swa_cache_write afterwards)."""
    torch = _torch()
    dt = _dtype_of(params)
    C = q.shape[1]
    qshp = (params.batch, C, params.n_q_heads, params.head_dim)
    kshp = (params.batch, C, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    if out is None:
        out = torch.empty(qshp, dtype=dt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((params.batch, params.n_q_heads, C), dtype=torch.float32, device=q.device)
    need = swa_prefill_workspace_bytes(params, C)
    workspace = _workspace(need, q.device, workspace)
    st = getattr(library(), _entry)(
        ctypes.byref(params), _ptr(q, "q", dt, qshp), _ptr(k, "k", dt, kshp), _ptr(v, "v", dt, kshp),
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp),
        _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), C,
        _ptr(out, "out", dt, qshp),
        _ptr(lse, "lse", torch.float32, (params.batch, params.n_q_heads, C)),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, _entry)
    return out, lse


def swa_prefill_chunk_aligned(params, q, k, v, k_cache, v_cache, start_pos, out=None, lse=None,
                              workspace=None, want_lse=True, stream=None):
    """swa_prefill_chunk for chunks whose starts are all multiples of the
    window (a prompt cut into chunks of W tokens); a sequence whose start is
    not gets NaN outputs.  Same arguments and results as swa_prefill_chunk."""
    return swa_prefill_chunk(params, q, k, v, k_cache, v_cache, start_pos, out, lse, workspace,
                             want_lse, stream, _entry="swa_prefill_chunk_aligned")


def swa_prefill_chunk_aligned_write_prev(params, k_prev, v_prev, start_prev, q, k, v, k_cache, v_cache,
                                         start_pos, out=None, lse=None, workspace=None, want_lse=True,
                                         stream=None):
    """swa_cache_write of the previous chunk (k_prev, v_prev from start_prev),
    then swa_prefill_chunk_aligned of the next (q, k, v from start_pos), with
    the write and the next chunk's key rotation in one pass; returns (out, lse)."""
    torch = _torch()
    dt = _dtype_of(params)
    C, Cp = q.shape[1], k_prev.shape[1]
    qshp = (params.batch, C, params.n_q_heads, params.head_dim)
    kshp = (params.batch, C, params.n_kv_heads, params.head_dim)
    pshp = (params.batch, Cp, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    if out is None:
        out = torch.empty(qshp, dtype=dt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((params.batch, params.n_q_heads, C), dtype=torch.float32, device=q.device)
    workspace = _workspace(swa_prefill_workspace_bytes(params, C), q.device, workspace)
    st = library().swa_prefill_chunk_aligned_write_prev(
        ctypes.byref(params), _ptr(k_prev, "k_prev", dt, pshp), _ptr(v_prev, "v_prev", dt, pshp),
        _ptr(start_prev, "start_prev", torch.int32, (params.batch,)), Cp,
        _ptr(q, "q", dt, qshp), _ptr(k, "k", dt, kshp), _ptr(v, "v", dt, kshp),
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp),
        _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), C,
        _ptr(out, "out", dt, qshp),
        _ptr(lse, "lse", torch.float32, (params.batch, params.n_q_heads, C)),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "swa_prefill_chunk_aligned_write_prev")
    return out, lse


def swa_rope_keys(params, k, start_pos, k_rot=None, stream=None):
    """Rotate keys k [B][n_tok][Hkv][D] at positions start_pos[b] + t; returns k_rot."""
    torch = _torch()
    dt = _dtype_of(params)
    shp = (params.batch, k.shape[1], params.n_kv_heads, params.head_dim)
    if k_rot is None:
        k_rot = torch.empty(shp, dtype=dt, device=k.device)
    st = library().swa_rope_keys(ctypes.byref(params), _ptr(k, "k", dt, shp),
                                 _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), k.shape[1],
                                 _ptr(k_rot, "k_rot", dt, shp), _stream(stream))
    _check(st, "swa_rope_keys")
    return k_rot


def swa_rope_keys_cache_write(params, k, v, start_pos, k_cache, v_cache, k_rot=None, stream=None):
    """swa_rope_keys and swa_cache_write in one pass, for a chunk whose
    attention reads no cache (a sequence's first chunk); returns k_rot."""
    torch = _torch()
    dt = _dtype_of(params)
    n_tok = k.shape[1]
    shp = (params.batch, n_tok, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    if k_rot is None:
        k_rot = torch.empty(shp, dtype=dt, device=k.device)
    st = library().swa_rope_keys_cache_write(
        ctypes.byref(params), _ptr(k, "k", dt, shp), _ptr(v, "v", dt, shp),
        _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), n_tok, _ptr(k_rot, "k_rot", dt, shp),
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp), _stream(stream))
    _check(st, "swa_rope_keys_cache_write")
    return k_rot


def swa_prefill_attention(params, q, k_rot, v, k_cache, v_cache, start_pos, out=None, lse=None,
                          want_lse=True, stream=None):
    """Attention pass of a prefill chunk over already-rotated keys; returns (out, lse)."""
    torch = _torch()
    dt = _dtype_of(params)
    C = q.shape[1]
    qshp = (params.batch, C, params.n_q_heads, params.head_dim)
    kshp = (params.batch, C, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    if out is None:
        out = torch.empty(qshp, dtype=dt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((params.batch, params.n_q_heads, C), dtype=torch.float32, device=q.device)
    st = library().swa_prefill_attention(
        ctypes.byref(params), _ptr(q, "q", dt, qshp), _ptr(k_rot, "k_rot", dt, kshp),
        _ptr(v, "v", dt, kshp), _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp),
        _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), C, _ptr(out, "out", dt, qshp),
        _ptr(lse, "lse", torch.float32, (params.batch, params.n_q_heads, C)), _stream(stream))
    _check(st, "swa_prefill_attention")
    return out, lse


def swa_decode(params, q, k_cache, v_cache, pos, out=None, lse=None, workspace=None,
               want_lse=True, stream=None):
    """One decode step per sequence (the cache must already hold pos[b]);
    returns (out, lse)."""
    torch = _torch()
    dt = _dtype_of(params)
    qshp = (params.batch, params.n_q_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    if out is None:
        out = torch.empty(qshp, dtype=dt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((params.batch, params.n_q_heads), dtype=torch.float32, device=q.device)
    need = swa_decode_workspace_bytes(params)
    workspace = _workspace(need, q.device, workspace)
    st = library().swa_decode(
        ctypes.byref(params), _ptr(q, "q", dt, qshp), _ptr(k_cache, "k_cache", dt, cshp),
        _ptr(v_cache, "v_cache", dt, cshp), _ptr(pos, "pos", torch.int32, (params.batch,)),
        _ptr(out, "out", dt, qshp), _ptr(lse, "lse", torch.float32, (params.batch, params.n_q_heads)),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "swa_decode")
    return out, lse


def swa_decode_step(params, q, k, v, k_cache, v_cache, pos, out=None, lse=None, workspace=None,
                    want_lse=True, stream=None):
    """One whole decode step per sequence: stores the new token's k/v
    ([B][Hkv][D], raw) at slot(pos[b]) of the caches, then attends; returns
    (out, lse)."""
    torch = _torch()
    dt = _dtype_of(params)
    qshp = (params.batch, params.n_q_heads, params.head_dim)
    kshp = (params.batch, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    if out is None:
        out = torch.empty(qshp, dtype=dt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((params.batch, params.n_q_heads), dtype=torch.float32, device=q.device)
    need = swa_decode_workspace_bytes(params)
    workspace = _workspace(need, q.device, workspace)
    st = library().swa_decode_step(
        ctypes.byref(params), _ptr(q, "q", dt, qshp), _ptr(k, "k", dt, kshp), _ptr(v, "v", dt, kshp),
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp),
        _ptr(pos, "pos", torch.int32, (params.batch,)),
        _ptr(out, "out", dt, qshp), _ptr(lse, "lse", torch.float32, (params.batch, params.n_q_heads)),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "swa_decode_step")
    return out, lse


def swa_noalloc_scratch_bytes() -> int:
    return int(library().swa_noalloc_scratch_bytes())


def swa_decode_step_noalloc(params, q, k, v, k_cache, v_cache, pos, out, lse=None, stream=None):
    """swa_decode_step with the library's fixed scratch array instead of a
    workspace: allocates nothing (out, and lse if wanted, are the caller's)."""
    torch = _torch()
    dt = _dtype_of(params)
    qshp = (params.batch, params.n_q_heads, params.head_dim)
    kshp = (params.batch, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    st = library().swa_decode_step_noalloc(
        ctypes.byref(params), _ptr(q, "q", dt, qshp), _ptr(k, "k", dt, kshp), _ptr(v, "v", dt, kshp),
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp),
        _ptr(pos, "pos", torch.int32, (params.batch,)),
        _ptr(out, "out", dt, qshp), _ptr(lse, "lse", torch.float32, (params.batch, params.n_q_heads)),
        _stream(stream))
    _check(st, "swa_decode_step_noalloc")
    return out, lse


def _lens(params, chunk_lens):
    """Host int32 array of the batch's chunk lengths (kept alive by the caller)
    and their total."""
    chunk_lens = [int(x) for x in chunk_lens]
    if len(chunk_lens) != params.batch:
        raise ValueError(f"chunk_lens has {len(chunk_lens)} entries, expected {params.batch}")
    return (ctypes.c_int32 * params.batch)(*chunk_lens), sum(chunk_lens)


def swa_prefill_varlen_workspace_bytes(params, chunk_lens) -> int:
    lens, _ = _lens(params, chunk_lens)
    return int(library().swa_prefill_varlen_workspace_bytes(ctypes.byref(params), lens))


def swa_rope_keys_varlen(params, k, start_pos, chunk_lens, k_rot=None, stream=None):
    """Packed keys [total][Hkv][D] rotated at their positions; returns k_rot."""
    torch = _torch()
    dt = _dtype_of(params)
    lens, total = _lens(params, chunk_lens)
    kshp = (total, params.n_kv_heads, params.head_dim)
    if k_rot is None:
        k_rot = torch.empty(kshp, dtype=dt, device=k.device)
    st = library().swa_rope_keys_varlen(
        ctypes.byref(params), _ptr(k, "k", dt, kshp), _ptr(start_pos, "start_pos", torch.int32, (params.batch,)),
        lens, _ptr(k_rot, "k_rot", dt, kshp), _stream(stream))
    _check(st, "swa_rope_keys_varlen")
    return k_rot


def swa_prefill_attention_varlen(params, q, k_rot, v, k_cache, v_cache, start_pos, chunk_lens, out=None,
                                 lse=None, want_lse=True, stream=None):
    """Attention of packed chunks of their own lengths; returns (out [total][Hq][D],
    lse [Hq][total])."""
    torch = _torch()
    dt = _dtype_of(params)
    lens, total = _lens(params, chunk_lens)
    qshp = (total, params.n_q_heads, params.head_dim)
    kshp = (total, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    if out is None:
        out = torch.empty(qshp, dtype=dt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((params.n_q_heads, total), dtype=torch.float32, device=q.device)
    st = library().swa_prefill_attention_varlen(
        ctypes.byref(params), _ptr(q, "q", dt, qshp), _ptr(k_rot, "k_rot", dt, kshp), _ptr(v, "v", dt, kshp),
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp),
        _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), lens,
        _ptr(out, "out", dt, qshp), _ptr(lse, "lse", torch.float32, (params.n_q_heads, total)), _stream(stream))
    _check(st, "swa_prefill_attention_varlen")
    return out, lse


def swa_prefill_chunk_varlen(params, q, k, v, k_cache, v_cache, start_pos, chunk_lens, out=None, lse=None,
                             workspace=None, want_lse=True, stream=None):
    """Key rotation + attention of packed chunks of their own lengths (the
    cache is not written); returns (out [total][Hq][D], lse [Hq][total])."""
    torch = _torch()
    dt = _dtype_of(params)
    lens, total = _lens(params, chunk_lens)
    qshp = (total, params.n_q_heads, params.head_dim)
    kshp = (total, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    if out is None:
        out = torch.empty(qshp, dtype=dt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((params.n_q_heads, total), dtype=torch.float32, device=q.device)
    need = int(library().swa_prefill_varlen_workspace_bytes(ctypes.byref(params), lens))
    workspace = _workspace(need, q.device, workspace)
    st = library().swa_prefill_chunk_varlen(
        ctypes.byref(params), _ptr(q, "q", dt, qshp), _ptr(k, "k", dt, kshp), _ptr(v, "v", dt, kshp),
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp),
        _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), lens,
        _ptr(out, "out", dt, qshp), _ptr(lse, "lse", torch.float32, (params.n_q_heads, total)),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "swa_prefill_chunk_varlen")
    return out, lse


def swa_cache_write_varlen(params, k, v, start_pos, chunk_lens, k_cache, v_cache, stream=None):
    """Packed k, v [total][Hkv][D] of chunks of their own lengths into the
    rolling buffers."""
    torch = _torch()
    dt = _dtype_of(params)
    lens, total = _lens(params, chunk_lens)
    kshp = (total, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    st = library().swa_cache_write_varlen(
        ctypes.byref(params), _ptr(k, "k", dt, kshp), _ptr(v, "v", dt, kshp),
        _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), lens,
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp), _stream(stream))
    _check(st, "swa_cache_write_varlen")


def swa_step_varlen_workspace_bytes(params, chunk_lens) -> int:
    lens, _ = _lens(params, chunk_lens)
    return int(library().swa_step_varlen_workspace_bytes(ctypes.byref(params), lens))


def swa_step_varlen(params, q, k, v, k_cache, v_cache, start_pos, chunk_lens, out=None, lse=None,
                    workspace=None, want_lse=True, stream=None):
    """One whole step of a mixed batch (attention of every packed chunk, the
    one-token sequences as decodes, then the cache write); returns (out
    [total][Hq][D], lse [Hq][total])."""
    torch = _torch()
    dt = _dtype_of(params)
    lens, total = _lens(params, chunk_lens)
    qshp = (total, params.n_q_heads, params.head_dim)
    kshp = (total, params.n_kv_heads, params.head_dim)
    cshp = (params.batch, params.n_sink + params.window, params.n_kv_heads, params.head_dim)
    if out is None:
        out = torch.empty(qshp, dtype=dt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((params.n_q_heads, total), dtype=torch.float32, device=q.device)
    need = int(library().swa_step_varlen_workspace_bytes(ctypes.byref(params), lens))
    workspace = _workspace(need, q.device, workspace)
    st = library().swa_step_varlen(
        ctypes.byref(params), _ptr(q, "q", dt, qshp), _ptr(k, "k", dt, kshp), _ptr(v, "v", dt, kshp),
        _ptr(k_cache, "k_cache", dt, cshp), _ptr(v_cache, "v_cache", dt, cshp),
        _ptr(start_pos, "start_pos", torch.int32, (params.batch,)), lens,
        _ptr(out, "out", dt, qshp), _ptr(lse, "lse", torch.float32, (params.n_q_heads, total)),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "swa_step_varlen")
    return out, lse


def swa_debug_slots(params, positions, stream=None):
    torch = _torch()
    slots = torch.empty_like(positions)
    st = library().swa_debug_slots(ctypes.byref(params), _ptr(positions, "positions", torch.int32),
                                   positions.numel(), _ptr(slots, "slots", torch.int32), _stream(stream))
    _check(st, "swa_debug_slots")
    return slots


def swa_debug_mask(params, q_pos, k_pos, stream=None):
    torch = _torch()
    mask = torch.empty(k_pos.shape, dtype=torch.uint8, device=k_pos.device)
    st = library().swa_debug_mask(ctypes.byref(params), int(q_pos), _ptr(k_pos, "k_pos", torch.int32),
                                  k_pos.numel(), _ptr(mask, "mask", torch.uint8), _stream(stream))
    _check(st, "swa_debug_mask")
    return mask
