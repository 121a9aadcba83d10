"""Slot-mapped K/V cache write and block copy-on-write — plain reference.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What is computed
----------------
Decoding token ``t`` computes only that token's K and V and appends them to
the cache ([KVPA] §2.2; [KV2P] §2.1).  With paging, the row goes to the last
block of the sequence's table at offset ``t % block_size`` ([KVPA] §5.3).  A
*slot* names that place as ``block * block_size + offset``; new token ``i``
is written to ``kv[slot // bs, 0, :, slot % bs, :] = key[i]`` and
``kv[slot // bs, 1, :, slot % bs, :] = value[i]`` for every KV head.

A sequence that is about to write into a block shared with another sequence
first gets a private copy of that block and repoints its table entry to it;
the other sequence keeps the original ([NANO] §2.3 fork example and §5.5;
[KVPA] §5.1 block manager with copy-on-write).  The copy is the whole block
(both K and V, every head, every row), taken before any new row is written.

Readings
--------
* A negative slot means "no write" for that row (the pages are silent).
* Copy pairs are applied in the order given, then the scatter; the block
  manager only emits pairs whose destination is a freshly taken block, so
  the order among pairs never matters for its output.
* The result is a byte copy: the output has the input's dtype and there is
  exactly one correct result.
"""

from __future__ import annotations

import numpy as np


def cache_write_ref(kv_cache, key, value, slot_mapping, cow_pairs=()):
    """Return a new pool with the copy-on-write copies and the scatter applied.

    kv_cache:     [NB, 2, Hkv, bs, D]
    key, value:   [T, Hkv, D], same dtype as the pool
    slot_mapping: [T] integer slots (negative = skip)
    cow_pairs:    iterable of (src_block, dst_block)
    """
    out = np.array(kv_cache, copy=True)
    block_size = out.shape[3]
    for src, dst in cow_pairs:
        out[int(dst)] = out[int(src)]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        out[block, 0, :, offset, :] = key[i]
        out[block, 1, :, offset, :] = value[i]
    return out
