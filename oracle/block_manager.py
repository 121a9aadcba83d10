"""Host block manager — a plain dict/list model.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What is modelled
----------------
The block manager owns a pool of fixed-size physical KV blocks and, per
sequence, a block table mapping logical block ``i`` to a physical block
([KVPA] §4.2 and §5.1-§5.3; [KV2P] §3.2 and the ``PagedKVCache`` of §6.2;
[NANO] §2.3 and the ``BlockManager`` of §4.2).

* Free pool: a list used as a stack.  It starts as ``[0, 1, ..., NB-1]``,
  takes from the end and returns to the end, as the ``PagedKVCache`` of
  [KV2P] §6.2 does with ``pop()`` / ``append``.  ([NANO] §4.2 takes from the
  front instead; block ids are policy, not semantics, and this model and the
  native manager share the stack policy so ids can be compared exactly.)
* Every physical block has a reference count: the number of sequence tables
  that hold it ([NANO] §2.3; [KVPA] §8.2-§8.3).  A block returns to the free
  pool when its count drops to 0.
* ``allocate(seq, n)``: ``ceil(n / bs)`` fresh blocks, count 1 each
  ([KV2P] §6.2 ``allocate``).  All or nothing: if too few blocks are free,
  nothing changes and an out-of-blocks error is raised ([KV2P] §6.2 raises,
  [NANO] §4.2 asserts).
* ``share(seq, blocks, n)``: extend a table with blocks that other sequences
  already hold and add one reference to each (prefix reuse, [KVPA] §8.2).
* ``fork(parent, child)``: the child's table is a copy of the parent's and
  every block gains a reference ([NANO] §2.3, sequence B forking from A).
* ``append_slot(seq)``: the place of the sequence's next token.  With ``t``
  tokens already held, a new block is taken when ``t % bs == 0``
  ([KVPA] §5.3: blocks needed = ceil((t+1)/bs)).  Otherwise the row goes into
  the last block; if that block is shared (count > 1) the sequence first
  takes a fresh block, drops one reference on the old one, repoints its last
  table entry and reports the (old, new) pair so the device copies the data
  ([NANO] §2.3 and §5.5, copy-on-write).  The slot is
  ``last_block * bs + t % bs``.
* ``free(seq)``: drop one reference per table entry, in table order, and
  return blocks that reach 0 ([KVPA] §8.2 step 3; [NANO] §4.2 ``free``).

Readings: an unknown or already-freed sequence is an error with no state
change ([NANO] §4.2 would raise ``KeyError``; [KV2P] §6.2 silently ignores).

Prefix cache (optional, ``enable_prefix_cache``)
-----------------------------------------------
Requests that start with the same tokens reuse the blocks that hold them
([KVPA] §8.1-§8.2: hash the prefix, look it up in a global cache, add a
reference to each reused block; [KV2P] §4.2: one hash per block from its
content and position, match block by block for the longest prefix, keep
reference counts, evict with LRU but never a referenced block; [NANO] §3.2:
hash fixed-size chunks so that partial matches count, §4.3: a dict from the
chunk hash to the block, reuse only full blocks).

* Block hash: ``h_i = FNV-1a-64(le64(h_{i-1}) || le32(t) for the bs token ids
  of block i)`` with ``h_{-1} = 0``, so a block's hash depends on its tokens
  and on everything before it (its position).  A match also compares the
  stored parent hash and token ids, so a hash collision is never a hit.
* ``allocate_prompt(seq, tokens)``: walk the prompt's full blocks from the
  start while their hashes are in the cache; every matched block gains a
  reference (and a hit); the rest of the prompt gets fresh blocks.  Returns
  the number of leading tokens whose K/V the matched blocks already hold.
* ``register(seq)``: after the caller wrote the K/V of the sequence's full
  blocks, put those not yet cached into the cache (a hash already present
  keeps its block; the sequence's copy stays private).  ``record_tokens``
  appends the ids of the tokens appended since the known ids ended (they
  must bring the known ids up to the tokens held), so that decoded blocks can
  be registered too.
* A cached block whose count drops to 0 is not returned to the free pool: it
  becomes evictable, stamped with a release clock.  Fresh blocks come from
  the free pool first; only when it is empty is an evictable block evicted
  (removed from the cache): the least recently released one, taking blocks
  with at least ``protect_hits`` hits last ([KV2P] §4.3: protect frequently
  reused prefixes against one-off requests; 0 = plain LRU).
* Admission threshold ``admit_after`` ([KV2P] §4.3, the other remedy for
  cache pollution: a prefix seen fewer times than a minimum does not enter
  the cache).  Reading: a full block is cached at registration only once its
  key (the chain hash, i.e. its tokens and position) has been registered
  ``admit_after`` times; the earlier copies stay private.  The keys still
  below the threshold and their counts are kept for at most ``num_blocks``
  keys, the one seen least recently dropped first.  1 (the default) caches
  at the first registration.
* With the cache on, ``free`` counts free plus evictable blocks.
"""

from __future__ import annotations

from collections import OrderedDict

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data, h=FNV_OFFSET):
    """64-bit FNV-1a over ``data`` (bytes), from its published definition:
    for each octet, xor it into the hash, then multiply by the FNV prime."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(parent, tokens):
    """Hash of one full block: its parent's hash (8 bytes, little endian)
    followed by its token ids (4 bytes each, little endian, two's complement)."""
    data = int(parent).to_bytes(8, "little") + b"".join(
        (int(t) & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    return fnv1a64(data)


class BlockManagerError(Exception):
    """Raised with ``kind`` in {"oom", "not_found", "invalid"}; state unchanged."""

    def __init__(self, kind, message):
        super().__init__(message)
        self.kind = kind


class BlockManagerModel:
    def __init__(self, num_blocks, block_size):
        if num_blocks <= 0 or block_size <= 0:
            raise BlockManagerError("invalid", "num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free_blocks = list(range(self.num_blocks))
        self.ref_counts = [0] * self.num_blocks
        self.tables = {}       # seq -> list of physical block ids
        self.num_tokens = {}   # seq -> tokens held
        # prefix cache
        self.cache_on = False
        self.protect_hits = 0
        self.admit_after = 1
        self.sightings = OrderedDict()   # key -> registrations, least recent first
        self.cache = {}        # hash -> block
        self.block_key = {}    # cached block -> (hash, parent hash, tokens)
        self.hits = [0] * self.num_blocks
        self.evictable = {}    # block -> (protected, release clock)
        self.clock = 0
        self.tokens = {}       # seq -> known token ids (a prefix of its tokens)
        self.registered = {}   # seq -> leading blocks already in the cache chain
        self.counters = {"lookups": 0, "hit_blocks": 0, "miss_blocks": 0, "evictions": 0,
                         "held_back": 0}

    # -- helpers -----------------------------------------------------------
    def _need(self, seq):
        if seq not in self.tables:
            raise BlockManagerError("not_found", f"unknown sequence {seq}")

    def _available(self):
        return len(self.free_blocks) + len(self.evictable)

    def _take(self):
        if self.free_blocks:
            block = self.free_blocks.pop()
        else:  # evict the least recently released, unprotected first
            block = min(self.evictable, key=lambda b: self.evictable[b])
            del self.evictable[block]
            h = self.block_key.pop(block)[0]
            del self.cache[h]
            self.hits[block] = 0
            self.counters["evictions"] += 1
        self.ref_counts[block] = 1
        return block

    def _release(self, block):
        self.ref_counts[block] -= 1
        if self.ref_counts[block] == 0:
            if block in self.block_key:
                prot = self.protect_hits > 0 and self.hits[block] >= self.protect_hits
                self.evictable[block] = (prot, self.clock)
                self.clock += 1
            else:
                self.free_blocks.append(block)

    # -- operations --------------------------------------------------------
    def allocate(self, seq, num_tokens):
        if seq in self.tables:
            raise BlockManagerError("invalid", f"sequence {seq} already exists")
        if num_tokens < 0:
            raise BlockManagerError("invalid", "negative token count")
        needed = -(-num_tokens // self.block_size)
        if self._available() < needed:
            raise BlockManagerError("oom", "out of KV cache blocks")
        self.tables[seq] = [self._take() for _ in range(needed)]
        self.num_tokens[seq] = num_tokens
        self.tokens[seq] = []
        self.registered[seq] = 0
        return list(self.tables[seq])

    def share(self, seq, blocks, num_tokens):
        blocks = [int(b) for b in blocks]
        if num_tokens < 0 or -(-num_tokens // self.block_size) != len(blocks):
            raise BlockManagerError("invalid", "token count does not match the shared blocks")
        for b in blocks:
            if not (0 <= b < self.num_blocks) or self.ref_counts[b] == 0:
                raise BlockManagerError("invalid", f"block {b} is not held by any sequence")
        if seq in self.tables and self.num_tokens[seq] % self.block_size:
            raise BlockManagerError("invalid", "sequence ends inside a block")
        table = self.tables.setdefault(seq, [])
        self.num_tokens.setdefault(seq, 0)
        self.tokens.setdefault(seq, [])
        self.registered.setdefault(seq, 0)
        for b in blocks:
            self.ref_counts[b] += 1
            table.append(b)
        self.num_tokens[seq] += num_tokens

    def fork(self, parent, child):
        self._need(parent)
        if child in self.tables:
            raise BlockManagerError("invalid", f"sequence {child} already exists")
        self.tables[child] = list(self.tables[parent])
        self.num_tokens[child] = self.num_tokens[parent]
        self.tokens[child] = list(self.tokens[parent])
        self.registered[child] = self.registered[parent]
        for b in self.tables[child]:
            self.ref_counts[b] += 1

    def append_slot(self, seq):
        """Returns (slot, cow_src, cow_dst); cow_* are -1 when no copy is needed."""
        self._need(seq)
        table = self.tables[seq]
        t = self.num_tokens[seq]
        offset = t % self.block_size
        cow_src = cow_dst = -1
        if offset == 0:
            if not self._available():
                raise BlockManagerError("oom", "out of KV cache blocks")
            table.append(self._take())
        elif self.ref_counts[table[-1]] > 1:
            if not self._available():
                raise BlockManagerError("oom", "out of KV cache blocks")
            old = table[-1]
            new = self._take()
            self.ref_counts[old] -= 1  # still > 0: another sequence holds it
            table[-1] = new
            cow_src, cow_dst = old, new
        self.num_tokens[seq] = t + 1
        return table[-1] * self.block_size + offset, cow_src, cow_dst

    def free(self, seq):
        self._need(seq)
        for b in self.tables.pop(seq):
            self._release(b)
        del self.num_tokens[seq]
        del self.tokens[seq]
        del self.registered[seq]

    # -- prefix cache ------------------------------------------------------
    def enable_prefix_cache(self, protect_hits=0, admit_after=1):
        if self.tables or protect_hits < 0 or admit_after < 1:
            raise BlockManagerError("invalid", "enable the prefix cache on an empty manager")
        self.cache_on = True
        self.protect_hits = int(protect_hits)
        self.admit_after = int(admit_after)

    def _admission_capacity(self):
        """Keys below the admission threshold remembered at most."""
        return self.num_blocks

    def _chain(self, seq, upto):
        """Hashes of the sequence's first ``upto`` full blocks."""
        toks, bs, h, out = self.tokens[seq], self.block_size, 0, []
        for i in range(upto):
            h = block_hash(h, toks[i * bs:(i + 1) * bs])
            out.append(h)
        return out

    def allocate_prompt(self, seq, tokens):
        """Returns (table, cached_tokens)."""
        if not self.cache_on:
            raise BlockManagerError("invalid", "prefix cache is off")
        if seq in self.tables:
            raise BlockManagerError("invalid", f"sequence {seq} already exists")
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        matched, parent = [], 0
        for i in range(len(tokens) // bs):
            blk = tokens[i * bs:(i + 1) * bs]
            h = block_hash(parent, blk)
            b = self.cache.get(h)
            if b is None or self.block_key[b][1:] != (parent, blk):
                break
            matched.append(b)
            parent = h
        needed = -(-len(tokens) // bs) - len(matched)
        if self._available() - sum(1 for b in matched if b in self.evictable) < needed:
            raise BlockManagerError("oom", "out of KV cache blocks")
        self.counters["lookups"] += 1
        self.counters["hit_blocks"] += len(matched)
        self.counters["miss_blocks"] += len(tokens) // bs - len(matched)
        for b in matched:
            if self.ref_counts[b] == 0:
                del self.evictable[b]
            self.ref_counts[b] += 1
            self.hits[b] += 1
        table = matched + [self._take() for _ in range(needed)]
        self.tables[seq] = table
        self.num_tokens[seq] = len(tokens)
        self.tokens[seq] = tokens
        self.registered[seq] = len(matched)
        return list(table), len(matched) * bs

    def record_tokens(self, seq, ids):
        self._need(seq)
        ids = [int(t) for t in ids]
        if len(self.tokens[seq]) + len(ids) != self.num_tokens[seq]:
            raise BlockManagerError("invalid", "token ids must complete the known prefix")
        self.tokens[seq].extend(ids)

    def register(self, seq):
        """Put the sequence's known full blocks into the cache; returns how
        many blocks were newly cached."""
        self._need(seq)
        if not self.cache_on:
            raise BlockManagerError("invalid", "prefix cache is off")
        full = len(self.tokens[seq]) // self.block_size
        hashes = self._chain(seq, full)
        added = 0
        for i in range(self.registered[seq], full):
            b = self.tables[seq][i]
            h = hashes[i]
            if h not in self.cache and b not in self.block_key:
                if self.admit_after > 1:
                    seen = self.sightings.pop(h, 0) + 1
                    if seen < self.admit_after:      # below the threshold: stays private
                        self.sightings[h] = seen
                        while len(self.sightings) > self._admission_capacity():
                            self.sightings.popitem(last=False)
                        self.counters["held_back"] += 1
                        continue
                parent = hashes[i - 1] if i else 0
                toks = self.tokens[seq][i * self.block_size:(i + 1) * self.block_size]
                self.cache[h] = b
                self.block_key[b] = (h, parent, toks)
                added += 1
        self.registered[seq] = full
        return added

    def prefix_stats(self):
        """(cached, evictable, lookups, hit_blocks, miss_blocks, evictions,
        registrations held back by the admission threshold)."""
        c = self.counters
        return (len(self.block_key), len(self.evictable), c["lookups"], c["hit_blocks"],
                c["miss_blocks"], c["evictions"], c["held_back"])

    # -- queries -----------------------------------------------------------
    def block_table(self, seq):
        self._need(seq)
        return list(self.tables[seq]), self.num_tokens[seq]

    def ref_count(self, block):
        if not (0 <= block < self.num_blocks):
            raise BlockManagerError("invalid", "block id out of range")
        return self.ref_counts[block]

    def stats(self):
        """(free, used, shared): free counts evictable cached blocks too;
        used = count >= 1, shared = count >= 2."""
        used = sum(1 for c in self.ref_counts if c >= 1)
        shared = sum(1 for c in self.ref_counts if c >= 2)
        return self._available(), used, shared
