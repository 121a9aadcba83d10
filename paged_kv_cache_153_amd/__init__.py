"""paged_kv_cache_153_amd — paged-KV decode attention for AMD MI355X (gfx950).

A thin ctypes binding over ``libpa.so`` (the C ABI declared in
``include/pa.h``).  This module only marshals arguments: it checks tensor
dtypes/shapes, passes raw device pointers and the current HIP stream, and
turns status codes into exceptions.  Every step of the computation runs in
the library's HIP kernels; there is no Python or CPU fallback, and a missing
library raises.

PyTorch supplies device memory and streams: outputs and split-context
workspaces the caller does not pass are allocated with ``torch.empty``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "PAError", "lib", "library_path", "cache_write", "decode", "decode_workspace_size", "prefill",
    "BlockManager", "KERNELS", "F32", "F16", "I8", "kv_scales_like",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpa.so")
_lib = None

F32, F16, I8 = 0, 1, 2
KERNELS = {"auto": 0, "valu": 1, "mfma": 2}
KV_CACHED = 0x100   # flag: plain cached K/V loads instead of streaming loads

PA_OK = 0
STATUS = {0: "PA_OK", -1: "PA_ERR_INVALID_ARG", -2: "PA_ERR_UNSUPPORTED", -3: "PA_ERR_WORKSPACE",
          -4: "PA_ERR_OOM", -5: "PA_ERR_NOT_FOUND", -6: "PA_ERR_HIP"}


class PAError(RuntimeError):
    def __init__(self, status, detail=""):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}" if detail else self.name)


def library_path():
    return _LIB_PATH


_c = ctypes
_P = _c.c_void_p
_I32P = _c.POINTER(_c.c_int32)
_I64P = _c.POINTER(_c.c_int64)

_SIGNATURES = {
    "pa_cache_write": (_c.c_int, [_P, _P, _P, _P, _P, _c.c_int64, _P, _c.c_int64, _c.c_int64,
                                  _c.c_int, _c.c_int, _c.c_int, _c.c_int, _P]),
    "pa_decode": (_c.c_int, [_P, _P, _P, _P, _P, _P, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                             _c.c_int, _c.c_int, _c.c_int, _c.c_int64, _c.c_float, _c.c_int,
                             _c.c_int, _c.c_int, _P, _c.c_size_t, _c.POINTER(_c.c_size_t),
                             _c.c_int, _P]),
    "pa_decode_static": (_c.c_int, [_P, _P, _P, _P, _P, _P, _c.c_int, _c.c_int, _c.c_int,
                                    _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int64,
                                    _c.c_float, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _P]),
    "pa_decode_static_capacity": (_c.c_size_t, []),
    "pa_prefill": (_c.c_int, [_P, _P, _P, _P, _P, _P, _P, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                              _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int64, _c.c_float,
                              _c.c_int, _c.c_int, _c.c_int, _P]),
    "pa_stage_from_host": (_c.c_int, [_P, _P, _c.c_int64, _P]),
    "pa_stage_and_write": (_c.c_int, [_P, _P, _c.c_int64, _P, _P, _P, _P, _P, _c.c_int64, _P,
                                      _c.c_int64, _c.c_int64, _c.c_int, _c.c_int, _c.c_int,
                                      _c.c_int, _P]),
    "pa_bm_create": (_P, [_c.c_int64, _c.c_int]),
    "pa_bm_destroy": (None, [_P]),
    "pa_bm_allocate": (_c.c_int, [_P, _c.c_int64, _c.c_int64]),
    "pa_bm_share": (_c.c_int, [_P, _c.c_int64, _I32P, _c.c_int, _c.c_int64]),
    "pa_bm_fork": (_c.c_int, [_P, _c.c_int64, _c.c_int64]),
    "pa_bm_append_slot": (_c.c_int, [_P, _c.c_int64, _I64P, _I32P, _I32P]),
    # the batched calls take buffer addresses as plain integers (no ctypes.cast)
    "pa_bm_append_slots": (_c.c_int, [_P, _P, _c.c_int, _P, _P,
                                      _c.POINTER(_c.c_int)]),
    "pa_bm_free": (_c.c_int, [_P, _c.c_int64]),
    "pa_bm_enable_prefix_cache": (_c.c_int, [_P, _c.c_int, _c.c_int]),
    "pa_bm_allocate_prompt": (_c.c_int, [_P, _c.c_int64, _I32P, _c.c_int64, _I64P]),
    "pa_bm_record_tokens": (_c.c_int, [_P, _c.c_int64, _I32P, _c.c_int64]),
    "pa_bm_register": (_c.c_int, [_P, _c.c_int64, _I64P]),
    "pa_bm_prefix_stats": (_c.c_int, [_P, _I64P]),
    "pa_bm_block_table": (_c.c_int, [_P, _c.c_int64, _I32P, _c.c_int, _c.POINTER(_c.c_int),
                                     _I64P]),
    "pa_bm_block_tables": (_c.c_int, [_P, _P, _c.c_int, _P, _c.c_int, _P]),
    "pa_bm_stats": (_c.c_int, [_P, _I64P, _I64P, _I64P]),
    "pa_bm_ref_count": (_c.c_int, [_P, _c.c_int32]),
    "pa_strerror": (_c.c_char_p, [_c.c_int]),
    "pa_last_error": (_c.c_char_p, []),
    "pa_version": (_c.c_char_p, []),
}


def lib():
    """Load ``libpa.so`` (built in-tree by ``build.py``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_153_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status):
    if status != PA_OK:
        detail = lib().pa_last_error().decode()
        raise PAError(status, detail)
    return status


# ---------------------------------------------------------------------------
# device calls
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.int8:
        return I8
    raise TypeError(f"unsupported dtype {t.dtype}")


def kv_scales_like(kv_cache):
    """A zeroed float32 scale array [NB, Hkv, 2, bs] for an INT8 pool."""
    torch = _torch()
    nb, two, hkv, bs, _ = kv_cache.shape
    return torch.zeros((nb, hkv, two, bs), dtype=torch.float32, device=kv_cache.device)


def _scales_ptr(kv_cache, kv_scales):
    """Pointer of the row-scale array an INT8 pool needs (None otherwise)."""
    torch = _torch()
    if kv_cache.dtype != torch.int8:
        if kv_scales is not None:
            raise TypeError("kv_scales is only for INT8 pools")
        return None
    nb, two, hkv, bs, _ = kv_cache.shape
    if kv_scales is None or kv_scales.dtype != torch.float32 or \
            tuple(kv_scales.shape) != (nb, hkv, two, bs):
        raise TypeError("an INT8 pool needs kv_scales float32 [NB, Hkv, 2, bs]")
    _need_cuda(kv_scales)
    return kv_scales.data_ptr()


def _stream(device, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return _P(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def stage_from_host(dst, src, stream=None):
    """Copy the page-locked host tensor ``src`` into the device tensor ``dst``
    (same number of bytes, both contiguous) with a kernel that reads the host
    buffer directly; enqueued on ``stream`` (default: the current stream)."""
    if not src.is_pinned() or src.is_cuda:
        raise TypeError("src must be a pinned host tensor")
    if not dst.is_cuda or not dst.is_contiguous() or not src.is_contiguous():
        raise TypeError("dst must be a contiguous device tensor and src contiguous")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src sizes differ")
    _check(lib().pa_stage_from_host(dst.data_ptr(), src.data_ptr(), nbytes,
                                    _stream(dst.device, stream)))
    return dst


def cache_write(key, value, kv_cache, slot_mapping, cow_pairs=None, stream=None,
                kv_scales=None):
    """Copy-on-write block copies (``cow_pairs`` [k, 2] int32 on device), then
    scatter ``key``/``value`` [T, Hkv, D] into ``kv_cache`` [NB, 2, Hkv, bs, D]
    at ``slot_mapping`` [T] int64 (negative = skip).  Enqueued on ``stream``.
    An int8 ``kv_cache`` takes float16 key/value rows, quantised per row into
    codes plus ``kv_scales`` [NB, Hkv, 2, bs] float32."""
    torch = _torch()
    _need_cuda(key, value, kv_cache, slot_mapping, cow_pairs)
    nb, two, hkv, bs, d = kv_cache.shape
    if two != 2 or key.shape != value.shape or key.dim() != 3 or key.shape[1:] != (hkv, d):
        raise ValueError("shape mismatch between key/value and kv_cache")
    in_dtype = torch.float16 if kv_cache.dtype == torch.int8 else kv_cache.dtype
    if key.dtype != in_dtype or value.dtype != in_dtype:
        raise TypeError("key and value must have the pool's dtype (float16 for an int8 pool)")
    sp = _scales_ptr(kv_cache, kv_scales)
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (key.shape[0],):
        raise TypeError("slot_mapping must be int64 [T]")
    ncow = 0
    if cow_pairs is not None:
        if cow_pairs.dtype != torch.int32 or cow_pairs.dim() != 2 or cow_pairs.shape[1] != 2:
            raise TypeError("cow_pairs must be int32 [k, 2]")
        ncow = cow_pairs.shape[0]
    _check(lib().pa_cache_write(key.data_ptr(), value.data_ptr(), kv_cache.data_ptr(), sp,
                                slot_mapping.data_ptr(), key.shape[0],
                                cow_pairs.data_ptr() if ncow else None, ncow, nb, hkv, d, bs,
                                _dtype_code(kv_cache), _stream(kv_cache.device, stream)))


def stage_and_write(stage_dst, stage_src, key, value, kv_cache, slot_mapping, cow_pairs=None,
                    stream=None, kv_scales=None):
    """``stage_from_host(stage_dst, stage_src)`` and ``cache_write(...)`` in one
    launch.  ``slot_mapping`` [T] int64 and ``cow_pairs`` [k, 2] int32 may be
    device tensors or pinned host tensors (for instance views into
    ``stage_src``), but not views into ``stage_dst``."""
    torch = _torch()
    _need_cuda(key, value, kv_cache, stage_dst)
    if not stage_src.is_pinned() or stage_src.is_cuda:
        raise TypeError("stage_src must be a pinned host tensor")
    if not stage_dst.is_contiguous() or not stage_src.is_contiguous():
        raise TypeError("stage_dst and stage_src must be contiguous")
    nbytes = stage_src.numel() * stage_src.element_size()
    if stage_dst.numel() * stage_dst.element_size() != nbytes:
        raise ValueError("stage_dst and stage_src sizes differ")
    for t in (slot_mapping, cow_pairs):
        if t is not None and not (t.is_cuda or t.is_pinned()):
            raise TypeError("slot_mapping / cow_pairs must be device or pinned host tensors")
    nb, two, hkv, bs, d = kv_cache.shape
    if two != 2 or key.shape != value.shape or key.dim() != 3 or key.shape[1:] != (hkv, d):
        raise ValueError("shape mismatch between key/value and kv_cache")
    in_dtype = torch.float16 if kv_cache.dtype == torch.int8 else kv_cache.dtype
    if key.dtype != in_dtype or value.dtype != in_dtype:
        raise TypeError("key and value must have the pool's dtype (float16 for an int8 pool)")
    sp = _scales_ptr(kv_cache, kv_scales)
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (key.shape[0],):
        raise TypeError("slot_mapping must be int64 [T]")
    ncow = 0
    if cow_pairs is not None:
        if cow_pairs.dtype != torch.int32 or cow_pairs.dim() != 2 or cow_pairs.shape[1] != 2:
            raise TypeError("cow_pairs must be int32 [k, 2]")
        ncow = cow_pairs.shape[0]
    _check(lib().pa_stage_and_write(stage_dst.data_ptr(), stage_src.data_ptr(), nbytes,
                                    key.data_ptr(), value.data_ptr(), kv_cache.data_ptr(), sp,
                                    slot_mapping.data_ptr(), key.shape[0],
                                    cow_pairs.data_ptr() if ncow else None, ncow, nb, hkv, d, bs,
                                    _dtype_code(kv_cache), _stream(kv_cache.device, stream)))
    return stage_dst


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, max_context_len, partition_size=0,
                          dtype=F16, kernel="auto", sliding_window=0, cached_kv=False):
    """Bytes of split-context workspace ``decode`` needs for this shape (the
    load policy ``cached_kv`` can change the schedule, hence the size)."""
    need = ctypes.c_size_t(0)
    _check(lib().pa_decode(None, None, None, None, None, None, num_seqs, num_q_heads,
                           num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len, 1, 1.0,
                           int(sliding_window), partition_size,
                           KERNELS[kernel] | (KV_CACHED if cached_kv else 0), None, 0,
                           ctypes.byref(need), dtype, None))
    return need.value


def decode(query, kv_cache, block_tables, context_lens, scale=None, max_context_len=None,
           partition_size=0, kernel="auto", out=None, workspace=None, stream=None,
           cached_kv=False, sliding_window=0, kv_scales=None):
    """Paged decode attention.

    query [S, Hq, D] (kv dtype), kv_cache [NB, 2, Hkv, bs, D], block_tables
    [S, MB] int32, context_lens [S] int32, all on the GPU.  Returns ``out``
    [S, Hq, D] float32.  ``max_context_len`` is a host bound on the lengths
    (default MB * bs); ``partition_size`` 0 = auto, -1 = single pass.
    ``cached_kv``: read K/V with cached loads (for pools whose blocks many
    sequences share); default streams them with non-temporal loads.
    ``sliding_window`` W > 0: each query attends to its sequence's last W
    tokens only; 0 = the whole context.  An int8 ``kv_cache`` needs its row
    scales ``kv_scales`` (written by ``cache_write``) and a float16 query.
    """
    torch = _torch()
    _need_cuda(query, kv_cache, block_tables, context_lens, out, workspace)
    nb, two, hkv, bs, d = kv_cache.shape
    s, hq, dq = query.shape
    if two != 2 or dq != d:
        raise ValueError("query/kv_cache shape mismatch")
    q_dtype = torch.float16 if kv_cache.dtype == torch.int8 else kv_cache.dtype
    if query.dtype != q_dtype:
        raise TypeError("query must have the pool's dtype (float16 for an int8 pool)")
    sp = _scales_ptr(kv_cache, kv_scales)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != s:
        raise TypeError("block_tables must be int32 [S, MB]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (s,):
        raise TypeError("context_lens must be int32 [S]")
    mb = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = mb * bs
    if scale is None:
        scale = d ** -0.5
    dt = _dtype_code(kv_cache)
    need = decode_workspace_size(s, hq, hkv, d, bs, mb, int(max_context_len), partition_size,
                                 dt, kernel, sliding_window, cached_kv)
    if out is None:
        out = torch.empty((s, hq, d), dtype=torch.float32, device=query.device)
    elif out.dtype != torch.float32 or out.shape != (s, hq, d):
        raise TypeError("out must be float32 [S, Hq, D]")
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode(out.data_ptr(), query.data_ptr(), kv_cache.data_ptr(), sp,
                           block_tables.data_ptr(), context_lens.data_ptr(), s, hq, hkv, d, bs,
                           mb, int(max_context_len), nb, float(scale), int(sliding_window),
                           int(partition_size),
                           KERNELS[kernel] | (KV_CACHED if cached_kv else 0),
                           None if workspace is None else workspace.data_ptr(),
                           wbytes, None, dt, _stream(query.device, stream)))
    return out


def decode_static(out, query, kv_cache, block_tables, context_lens, scale=None,
                  max_context_len=None, partition_size=0, kernel="auto", stream=None,
                  cached_kv=False, sliding_window=0, kv_scales=None):
    """``decode`` for callers that cannot allocate device memory: the caller
    passes ``out`` [S, Hq, D] float32, and the split-context partials go to
    the library's own per-GPU array (``pa_decode_static``; raises with
    PA_ERR_WORKSPACE when they need more than its
    ``pa_decode_static_capacity()`` bytes).  Calls that overlap on one GPU
    share that array and race."""
    torch = _torch()
    _need_cuda(out, query, kv_cache, block_tables, context_lens)
    nb, two, hkv, bs, d = kv_cache.shape
    s, hq, dq = query.shape
    if two != 2 or dq != d:
        raise ValueError("query/kv_cache shape mismatch")
    q_dtype = torch.float16 if kv_cache.dtype == torch.int8 else kv_cache.dtype
    if query.dtype != q_dtype:
        raise TypeError("query must have the pool's dtype (float16 for an int8 pool)")
    sp = _scales_ptr(kv_cache, kv_scales)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != s:
        raise TypeError("block_tables must be int32 [S, MB]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (s,):
        raise TypeError("context_lens must be int32 [S]")
    if out.dtype != torch.float32 or out.shape != (s, hq, d):
        raise TypeError("out must be float32 [S, Hq, D]")
    mb = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = mb * bs
    if scale is None:
        scale = d ** -0.5
    _check(lib().pa_decode_static(out.data_ptr(), query.data_ptr(), kv_cache.data_ptr(), sp,
                                  block_tables.data_ptr(), context_lens.data_ptr(), s, hq, hkv, d,
                                  bs, mb, int(max_context_len), nb, float(scale),
                                  int(sliding_window), int(partition_size),
                                  KERNELS[kernel] | (KV_CACHED if cached_kv else 0),
                                  _dtype_code(kv_cache), _stream(query.device, stream)))
    return out


def prefill(query, kv_cache, block_tables, context_lens, query_start, scale=None,
            max_query_len=None, out=None, stream=None, sliding_window=0, kv_scales=None):
    """Causal attention of multi-token query chunks over the paged cache.

    query [total_q, Hq, D] float16 (the chunks of all sequences, in order),
    kv_cache [NB, 2, Hkv, bs, D] float16 with the chunks' K/V already written,
    block_tables [S, MB] int32, context_lens [S] int32 (chunks included),
    query_start [S + 1] int32.  Query i of sequence s attends to the keys up
    to its own position n_s - T_s + i (with ``sliding_window`` W > 0, only
    the last W of them).  Returns ``out`` [total_q, Hq, D] float32.
    ``max_query_len`` is a host bound on the chunk lengths (default total_q).
    An int8 ``kv_cache`` needs its row scales ``kv_scales`` (written by
    ``cache_write``).
    """
    torch = _torch()
    _need_cuda(query, kv_cache, block_tables, context_lens, query_start, out)
    nb, two, hkv, bs, d = kv_cache.shape
    total, hq, dq = query.shape
    s = block_tables.shape[0]
    if two != 2 or dq != d:
        raise ValueError("query/kv_cache shape mismatch")
    if query.dtype != torch.float16 or kv_cache.dtype not in (torch.float16, torch.int8):
        raise TypeError("prefill takes a float16 query and a float16 or int8 pool")
    sp = _scales_ptr(kv_cache, kv_scales)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or \
            query_start.dtype != torch.int32 or context_lens.shape != (s,) or \
            query_start.shape != (s + 1,):
        raise TypeError("block_tables [S, MB], context_lens [S] and query_start [S+1] must be int32")
    if scale is None:
        scale = d ** -0.5
    if max_query_len is None:
        max_query_len = total
    if out is None:
        out = torch.empty((total, hq, d), dtype=torch.float32, device=query.device)
    elif out.dtype != torch.float32 or out.shape != (total, hq, d):
        raise TypeError("out must be float32 [total_q, Hq, D]")
    _check(lib().pa_prefill(out.data_ptr(), query.data_ptr(), kv_cache.data_ptr(), sp,
                            block_tables.data_ptr(), context_lens.data_ptr(),
                            query_start.data_ptr(), s, total, hq, hkv, d, bs,
                            block_tables.shape[1], int(max_query_len), nb, float(scale),
                            int(sliding_window), 0, _dtype_code(kv_cache),
                            _stream(query.device, stream)))
    return out


def _addr(t):
    """Address of a contiguous CPU tensor's data (no copy), as an integer for
    a ``c_void_p`` parameter."""
    if t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous CPU tensor")
    return t.data_ptr()


# ---------------------------------------------------------------------------
# host block manager
# ---------------------------------------------------------------------------
class BlockManager:
    """Handle over the native block manager (``pa_bm_*``; host memory only)."""

    def __init__(self, num_blocks, block_size):
        self._h = lib().pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise PAError(-1, lib().pa_last_error().decode())
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def allocate(self, seq, num_tokens):
        _check(lib().pa_bm_allocate(self._h, int(seq), int(num_tokens)))
        return self.block_table(seq)[0]

    def share(self, seq, blocks, num_tokens):
        arr = (ctypes.c_int32 * max(1, len(blocks)))(*[int(b) for b in blocks])
        _check(lib().pa_bm_share(self._h, int(seq), arr, len(blocks), int(num_tokens)))

    def fork(self, parent, child):
        _check(lib().pa_bm_fork(self._h, int(parent), int(child)))

    def append_slot(self, seq):
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_bm_append_slot(self._h, int(seq), ctypes.byref(slot), ctypes.byref(src),
                                       ctypes.byref(dst)))
        return slot.value, src.value, dst.value

    def append_slots(self, seqs):
        """Batched append: returns (slots list, [(src, dst), ...])."""
        n = len(seqs)
        sq = (ctypes.c_int64 * max(1, n))(*[int(x) for x in seqs])
        slots = (ctypes.c_int64 * max(1, n))()
        pairs = (ctypes.c_int32 * max(2, 2 * n))()
        k = ctypes.c_int(0)
        _check(lib().pa_bm_append_slots(self._h, sq, n, slots, pairs, ctypes.byref(k)))
        return list(slots[:n]), [(pairs[2 * i], pairs[2 * i + 1]) for i in range(k.value)]

    def free(self, seq):
        _check(lib().pa_bm_free(self._h, int(seq)))

    def block_table(self, seq):
        n, ntok = ctypes.c_int(0), ctypes.c_int64(0)
        _check(lib().pa_bm_block_table(self._h, int(seq), None, 0, ctypes.byref(n),
                                       ctypes.byref(ntok)))
        buf = (ctypes.c_int32 * max(1, n.value))()
        _check(lib().pa_bm_block_table(self._h, int(seq), buf, n.value, ctypes.byref(n),
                                       ctypes.byref(ntok)))
        return list(buf[:n.value]), ntok.value

    def num_tokens(self, seq):
        """Tokens of ``seq`` (its context length), without copying its table."""
        n, ntok = ctypes.c_int(0), ctypes.c_int64(0)
        _check(lib().pa_bm_block_table(self._h, int(seq), None, 0, ctypes.byref(n),
                                       ctypes.byref(ntok)))
        return ntok.value

    def block_tables(self, seqs, max_blocks):
        """Padded int32 tables [n, max_blocks] (-1 fill) and int32 lengths, as
        Python lists of rows (the caller copies them to the device)."""
        n = len(seqs)
        sq = (ctypes.c_int64 * max(1, n))(*[int(x) for x in seqs])
        tab = (ctypes.c_int32 * max(1, n * max_blocks))()
        lens = (ctypes.c_int32 * max(1, n))()
        _check(lib().pa_bm_block_tables(self._h, sq, n, tab, int(max_blocks), lens))
        rows = [list(tab[i * max_blocks:(i + 1) * max_blocks]) for i in range(n)]
        return rows, list(lens[:n])

    def append_slots_into(self, seqs, slots, cow_pairs):
        """Batched append writing straight into CPU tensors (e.g. pinned):
        ``seqs`` int64 [n], ``slots`` int64 [n], ``cow_pairs`` int32 [n, 2].
        Returns the number of copy pairs written."""
        n = seqs.numel()
        k = ctypes.c_int(0)
        _check(lib().pa_bm_append_slots(self._h, _addr(seqs), n, _addr(slots),
                                        _addr(cow_pairs), ctypes.byref(k)))
        return k.value

    def block_tables_into(self, seqs, tables, context_lens):
        """Fill CPU int32 ``tables`` [n, MB] (-1 padded) and ``context_lens`` [n]."""
        n = seqs.numel()
        _check(lib().pa_bm_block_tables(self._h, _addr(seqs), n, _addr(tables),
                                        tables.shape[1], _addr(context_lens)))

    def stats(self):
        f, u, s = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().pa_bm_stats(self._h, ctypes.byref(f), ctypes.byref(u), ctypes.byref(s)))
        return f.value, u.value, s.value

    def ref_count(self, block):
        r = lib().pa_bm_ref_count(self._h, int(block))
        if r < 0:
            _check(r)
        return r

    # -- prefix cache --------------------------------------------------------
    def enable_prefix_cache(self, protect_hits=0, admit_after=1):
        _check(lib().pa_bm_enable_prefix_cache(self._h, int(protect_hits), int(admit_after)))

    def allocate_prompt(self, seq, tokens):
        """Admit a prompt (token ids); returns (block table, cached_tokens)."""
        n = len(tokens)
        arr = (ctypes.c_int32 * max(1, n))(*[int(t) for t in tokens])
        cached = ctypes.c_int64(0)
        _check(lib().pa_bm_allocate_prompt(self._h, int(seq), arr, n, ctypes.byref(cached)))
        return self.block_table(seq)[0], cached.value

    def record_tokens(self, seq, tokens):
        n = len(tokens)
        arr = (ctypes.c_int32 * max(1, n))(*[int(t) for t in tokens])
        _check(lib().pa_bm_record_tokens(self._h, int(seq), arr, n))

    def register(self, seq):
        added = ctypes.c_int64(0)
        _check(lib().pa_bm_register(self._h, int(seq), ctypes.byref(added)))
        return added.value

    def prefix_stats(self):
        """(cached, evictable, lookups, hit_blocks, miss_blocks, evictions,
        held_back)."""
        out = (ctypes.c_int64 * 7)()
        _check(lib().pa_bm_prefix_stats(self._h, out))
        return tuple(out)
