"""INT8 KV cache with group-wise scales — plain reference.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What the pages say
------------------
[KV2P] §5.2 (quantisation trades precision for space): storing the KV cache in
INT8 instead of FP16 halves its size.  The page compares three ways to pick
the scale — one per tensor, one per channel, or one per group of elements
(128-element groups as the example), the last being the most accurate — and
§7.5 lists a quantised KV cache as the remedy when decode is limited by
memory bandwidth.  §7.4 adds that quantisation can be applied layer by layer.

Readings (the pages give no formula)
------------------------------------
* Group = the ``head_dim`` values of one token of one KV head, for K and for
  V separately: one group of 128 elements at head_dim 128 (the page's
  example), the whole 64-element row at head_dim 64.  Each group has its own
  float32 scale, stored beside the codes as ``scales[block, head, 0|1, row]``
  (the K and V scales of one block and head side by side).
* Symmetric quantisation: ``scale = amax / 127`` with ``amax = max |x|`` over
  the group, codes ``q = clamp(rint(x / scale), -127, 127)`` (round half to
  even), dequantised value ``q * scale``.  A group that is all zeros has
  scale 0 and codes 0.
* The codes are integers, so the decisions that make them are taken in
  float32 — the precision the GPU path computes them in: ``amax / 127`` and
  ``x / scale`` are correctly rounded float32 divisions of the float16 inputs
  widened to float32.  Dequantisation and everything after it is float64.
* Decode over an INT8 cache is decode attention over the dequantised cache:
  quantisation changes which values are stored, not what is computed.  The
  same holds for multi-token (chunked prefill) queries, which the page also
  runs over the cache ([KV2P] §5.4).
"""

from __future__ import annotations

import numpy as np

from .attention import decode_ref, prefill_ref

QMAX = 127


def quantize_rows_ref(x):
    """Quantise every row (last axis) of ``x`` to INT8 with its own scale.

    x:       [..., D] float16 or float32 values
    returns  (codes [..., D] int8, scales [...] float32)
    """
    xf = np.asarray(x).astype(np.float32)
    amax = np.max(np.abs(xf), axis=-1)
    scales = (amax / np.float32(QMAX)).astype(np.float32)
    codes = np.zeros(xf.shape, dtype=np.int8)
    live = scales > 0
    ratio = xf[live] / scales[live][..., None]          # float32 division
    codes[live] = np.clip(np.rint(ratio), -QMAX, QMAX).astype(np.int8)
    return codes, scales


def dequantize_ref(codes, scales):
    """``codes * scale`` per row, in float64 (exact: an int8 times a float32)."""
    return np.asarray(codes).astype(np.float64) * np.asarray(scales).astype(np.float64)[..., None]


def cache_write_i8_ref(kv_codes, kv_scales, key, value, slot_mapping, cow_pairs=()):
    """The slot-mapped write of ``cache.cache_write_ref`` into an INT8 pool.

    kv_codes:     [NB, 2, Hkv, bs, D] int8
    kv_scales:    [NB, Hkv, 2, bs] float32
    key, value:   [T, Hkv, D] float16
    slot_mapping: [T] (negative = skip); cow_pairs: (src, dst) block copies,
                  applied first, codes and scales alike
    returns       (new codes, new scales)
    """
    codes = np.array(kv_codes, copy=True)
    scales = np.array(kv_scales, copy=True)
    block_size = codes.shape[3]
    for src, dst in cow_pairs:
        codes[int(dst)] = codes[int(src)]
        scales[int(dst)] = scales[int(src)]
    kq, ks = quantize_rows_ref(key)
    vq, vs = quantize_rows_ref(value)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        codes[block, 0, :, offset, :] = kq[i]
        scales[block, :, 0, offset] = ks[i]
        codes[block, 1, :, offset, :] = vq[i]
        scales[block, :, 1, offset] = vs[i]
    return codes, scales


def decode_i8_ref(q, kv_codes, kv_scales, block_tables, context_lens, scale, window=0):
    """Decode attention over the dequantised INT8 pool (float64); scales
    [NB, Hkv, 2, bs] as ``cache_write_i8_ref`` writes them."""
    per_row = np.swapaxes(np.asarray(kv_scales), 1, 2)    # -> [NB, 2, Hkv, bs], as the codes
    return decode_ref(q, dequantize_ref(kv_codes, per_row), block_tables, context_lens, scale,
                      window=window)


def prefill_i8_ref(q, kv_codes, kv_scales, block_tables, context_lens, query_start, scale,
                   window=0):
    """Causal multi-token attention (``attention.prefill_ref``) over the
    dequantised INT8 pool (float64); scales [NB, Hkv, 2, bs]."""
    per_row = np.swapaxes(np.asarray(kv_scales), 1, 2)    # -> [NB, 2, Hkv, bs], as the codes
    return prefill_ref(q, dequantize_ref(kv_codes, per_row), block_tables, context_lens,
                       query_start, scale, window=window)
