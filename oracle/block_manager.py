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
"""

from __future__ import annotations


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

    # -- helpers -----------------------------------------------------------
    def _need(self, seq):
        if seq not in self.tables:
            raise BlockManagerError("not_found", f"unknown sequence {seq}")

    def _take(self):
        block = self.free_blocks.pop()
        self.ref_counts[block] = 1
        return block

    def _release(self, block):
        self.ref_counts[block] -= 1
        if self.ref_counts[block] == 0:
            self.free_blocks.append(block)

    # -- operations --------------------------------------------------------
    def allocate(self, seq, num_tokens):
        if seq in self.tables:
            raise BlockManagerError("invalid", f"sequence {seq} already exists")
        if num_tokens < 0:
            raise BlockManagerError("invalid", "negative token count")
        needed = -(-num_tokens // self.block_size)
        if len(self.free_blocks) < needed:
            raise BlockManagerError("oom", "out of KV cache blocks")
        self.tables[seq] = [self._take() for _ in range(needed)]
        self.num_tokens[seq] = num_tokens
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
            if not self.free_blocks:
                raise BlockManagerError("oom", "out of KV cache blocks")
            table.append(self._take())
        elif self.ref_counts[table[-1]] > 1:
            if not self.free_blocks:
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

    # -- queries -----------------------------------------------------------
    def block_table(self, seq):
        self._need(seq)
        return list(self.tables[seq]), self.num_tokens[seq]

    def ref_count(self, block):
        if not (0 <= block < self.num_blocks):
            raise BlockManagerError("invalid", "block id out of range")
        return self.ref_counts[block]

    def stats(self):
        """(free, used, shared): used = count >= 1, shared = count >= 2."""
        used = sum(1 for c in self.ref_counts if c >= 1)
        shared = sum(1 for c in self.ref_counts if c >= 2)
        return len(self.free_blocks), used, shared
