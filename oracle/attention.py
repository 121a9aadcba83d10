"""Decode attention over a paged KV cache — plain float64 definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``): imported by ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.

What is computed
----------------
For every sequence ``s`` and query head ``h`` the output is scaled dot-product
attention of one query row against the sequence's cached keys and values,
``softmax(scale * q K^T) V`` ([KVPA] §2.1, the attention formula; the decode
case has one query row and ``S`` cached rows).  The cached rows are not stored
contiguously: token ``t`` of a sequence sits in physical block
``block_table[t // block_size]`` at row ``t % block_size`` ([KVPA] §4.2, the
100-token / block-size-16 paging example and its block table; §5.3, where the
new token's row is ``t % block_size`` of the last block).

The physical pool has layout ``[num_blocks, 2, num_kv_heads, block_size,
head_dim]`` with index 0 = K and 1 = V ([KVPA] §4.3 and §5.1, the KV-cache
shape drawn for the kernel and the engine).

Readings where the pages are silent or inconsistent
---------------------------------------------------
* Only tokens ``t < context_len`` take part.  The page's block-level
  pseudocode multiplies whole blocks, but its own example says the last block
  is only partly filled ([KVPA] §4.2), so rows past the context are not keys.
* [KVPA] §4.3 normalises a softmax inside every block and sums the block
  outputs; that is not attention.  The global softmax of §2.1 is taken,
  which is also what the online-softmax loop of §7.2 reaches.
* Grouped-query attention ([KV2P] §5.3; [NANO] §1.2): query heads are split
  into ``num_kv_heads`` contiguous groups of ``G = Hq / Hkv``; query head
  ``h`` reads KV head ``h // G``.
* A sequence with context length 0 has output 0 (the pages' loop would end
  with 0/0).

Sliding window
--------------
[KV2P] §7.2 lists sliding-window attention among the remedies for long
contexts: each new token attends only to the last W tokens.  With
``window = W > 0`` the keys are tokens ``t`` with ``max(0, n - W) <= t < n``;
``window = 0`` means the whole context.

Multi-token queries (chunked prefill)
-------------------------------------
A prefill chunk brings T > 1 new tokens per sequence at once ([KV2P] §5.4:
a long prompt's prefill is split into chunks; [INFRA] §2: with T > 1 the
scores need a causal mask).  The chunk's K/V are written to the cache first;
query ``i`` of the chunk sits at position ``p = n - T + i`` and attends to the
keys ``t <= p``.  Reading: the page's mask is square (``tril(T, T)``) while
its scores span past + T keys; the plain reading is the mask aligned to the
end (each query sees all past tokens and the chunk tokens up to itself),
which for T = 1 is the decode case and for n = T is the square mask.

With a sliding window of W tokens (the remedy [KV2P] §7.2 names for long
contexts) each query sees only the last W tokens up to and including its own
position: keys ``max(0, p + 1 - W) <= t <= p``.  Reading: the decode's window
(the last W of the n cached tokens, the newest included) applied at every
query position of the chunk, so T = 1 is the windowed decode.

Split-context partials
----------------------
The pages merge block results with decay factors ([KVPA] §7.2 running max /
running sum; [NANO] §2.4 merging across blocks with decay coefficients).  The
same algebra across fixed-size token partitions gives, per partition ``p``,
``m_p = max z``, ``l_p = sum exp(z - m_p)``, ``o_p = sum exp(z - m_p) v / l_p``
and, across partitions, ``M = max m_p``, ``w_p = l_p exp(m_p - M)``,
``out = sum w_p o_p / sum w_p``.  ``split_ref`` and ``merge_ref`` write that
out; their agreement with ``decode_ref`` is a test.
"""

from __future__ import annotations

import numpy as np


def gather_sequence(kv_cache, block_table_row, context_len):
    """Return the logical K and V rows of one sequence, each ``[n, Hkv, D]``.

    Token ``t`` is read from physical block ``block_table_row[t // bs]``, row
    ``t % bs`` ([KVPA] §4.2 example: with block size 16, tokens 96..99 sit in
    the seventh table entry, rows 0..3).  Only ``t < context_len`` is read, so
    table entries past ``ceil(n / bs)`` and rows past ``n`` in the last block
    are never touched.
    """
    block_size = kv_cache.shape[3]
    t = np.arange(int(context_len))
    physical = np.asarray(block_table_row)[t // block_size]
    row = t % block_size
    # advanced indices separated by a slice: the token axis comes first
    k = kv_cache[physical, 0, :, row, :]
    v = kv_cache[physical, 1, :, row, :]
    return k, v


def _attend(qvec, keys, values, scale):
    """softmax(scale * keys @ q) @ values for one query row, in float64."""
    z = scale * (keys @ qvec)
    w = np.exp(z - z.max())
    return (w @ values) / w.sum()


def decode_ref(q, kv_cache, block_tables, context_lens, scale, window=0):
    """Reference decode attention.

    q:             [S, Hq, D]  (any float dtype; upcast exactly to float64)
    kv_cache:      [NB, 2, Hkv, bs, D]
    block_tables:  [S, max_blocks] integer, physical block ids
    context_lens:  [S] integer
    scale:         softmax scale (the pages use 1/sqrt(head_dim))
    window:        0 = whole context; W > 0 = only the last W tokens
    returns        [S, Hq, D] float64
    """
    q = np.asarray(q)
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = kv_cache.shape[2]
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        k, v = gather_sequence(kv_cache, block_tables[s], n)
        start = max(0, n - window) if window > 0 else 0
        k = k[start:].astype(np.float64)
        v = v[start:].astype(np.float64)
        for h in range(num_q_heads):
            g = h // group
            out[s, h] = _attend(q[s, h].astype(np.float64), k[:, g, :], v[:, g, :], scale)
    return out


def prefill_ref(q, kv_cache, block_tables, context_lens, query_start, scale, window=0):
    """Causal attention of multi-token queries over a paged cache.

    q:            [total_q, Hq, D], the queries of sequence s are rows
                  ``query_start[s] .. query_start[s+1]-1`` (T_s of them)
    context_lens: [S], n_s, counting the chunk (n_s >= T_s)
    query_start:  [S+1] increasing, query_start[0] = 0
    window:       0 = every earlier key; W > 0 = only the last W tokens up
                  to the query's own position
    returns       [total_q, Hq, D] float64: row ``query_start[s] + i`` is the
                  attention of query i over keys t <= p = n_s - T_s + i
                  (and t > p - W under a window)
    """
    q = np.asarray(q)
    total, num_q_heads, head_dim = q.shape
    num_kv_heads = kv_cache.shape[2]
    group = num_q_heads // num_kv_heads
    out = np.zeros((total, num_q_heads, head_dim), dtype=np.float64)
    for s in range(len(context_lens)):
        n = int(context_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        T = q1 - q0
        if T == 0:
            continue
        if T > n:
            raise ValueError("a chunk cannot be longer than its context")
        k, v = gather_sequence(kv_cache, block_tables[s], n)
        k = k.astype(np.float64)
        v = v.astype(np.float64)
        for i in range(T):
            p = n - T + i
            lo = max(0, p + 1 - window) if window > 0 else 0
            for h in range(num_q_heads):
                g = h // group
                out[q0 + i, h] = _attend(q[q0 + i, h].astype(np.float64), k[lo:p + 1, g, :],
                                         v[lo:p + 1, g, :], scale)
    return out


def split_ref(q, kv_cache, block_tables, context_lens, scale, partition_size):
    """Per-partition partial results of decode attention.

    Tokens of sequence ``s`` are cut into partitions of ``partition_size``
    logical tokens.  For partition ``p`` and head ``h``:
    ``m = max z``, ``l = sum exp(z - m)``, ``o = sum exp(z - m) v / l`` with
    ``z = scale * q.k`` over the partition's tokens.  Partitions with no token
    get ``m = -inf``, ``l = 0``, ``o = 0``.

    returns (m [S, Hq, NP], l [S, Hq, NP], o [S, Hq, NP, D]), float64, with
    ``NP = ceil(max(context_lens) / partition_size)``.
    """
    q = np.asarray(q)
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = kv_cache.shape[2]
    group = num_q_heads // num_kv_heads
    max_len = int(np.max(context_lens)) if len(context_lens) else 0
    num_parts = max(1, -(-max_len // partition_size))
    m = np.full((num_seqs, num_q_heads, num_parts), -np.inf)
    l = np.zeros((num_seqs, num_q_heads, num_parts))
    o = np.zeros((num_seqs, num_q_heads, num_parts, head_dim))
    for s in range(num_seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        k, v = gather_sequence(kv_cache, block_tables[s], n)
        k = k.astype(np.float64)
        v = v.astype(np.float64)
        for p in range(num_parts):
            lo, hi = p * partition_size, min(n, (p + 1) * partition_size)
            if lo >= hi:
                continue
            for h in range(num_q_heads):
                g = h // group
                z = scale * (k[lo:hi, g, :] @ q[s, h].astype(np.float64))
                m[s, h, p] = z.max()
                w = np.exp(z - m[s, h, p])
                l[s, h, p] = w.sum()
                o[s, h, p] = (w @ v[lo:hi, g, :]) / l[s, h, p]
    return m, l, o


def merge_ref(m, l, o):
    """Log-sum-exp merge of partition partials into the attention output.

    ``M = max_p m_p``; ``w_p = l_p exp(m_p - M)``; ``out = sum w_p o_p / sum w_p``.
    Empty partitions (``l_p = 0``) weigh nothing; if every partition is empty
    the output is 0.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    out = np.zeros(o.shape[:2] + o.shape[3:])
    for s in range(m.shape[0]):
        for h in range(m.shape[1]):
            live = l[s, h] > 0
            if not live.any():
                continue
            big = m[s, h, live].max()
            w = l[s, h, live] * np.exp(m[s, h, live] - big)
            out[s, h] = (w @ o[s, h, live]) / w.sum()
    return out
