"""Pins for the oracle's cache write and block-manager model.  CPU only."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth
from oracle import BlockManagerError, BlockManagerModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _example():
    with open(os.path.join(GOLDEN, "paging_example.json")) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Cache write: round trip through the page's paging example ([KVPA] §4.2, §5.3)
# --------------------------------------------------------------------------
def test_cache_write_round_trips_through_page_example():
    ex = _example()
    bs, n = ex["block_size"], ex["num_tokens"]
    rng = np.random.default_rng(0)
    pool = rng.standard_normal((10, 2, 3, bs, 8)).astype(np.float16)
    key = rng.standard_normal((n, 3, 8)).astype(np.float16)
    value = rng.standard_normal((n, 3, 8)).astype(np.float16)
    # slots straight from the printed ranges: physical block * 16 + row in block
    slots = np.empty(n, dtype=np.int64)
    for r in ex["ranges"]:
        lo, hi = r["tokens"]
        slots[lo:hi + 1] = r["physical"] * bs + np.arange(hi - lo + 1)
    out = oracle.cache_write_ref(pool, key, value, slots)
    k, v = oracle.gather_sequence(out, np.array(ex["block_table"]), n)
    assert np.array_equal(k.view(np.uint16), key.view(np.uint16))
    assert np.array_equal(v.view(np.uint16), value.view(np.uint16))
    # token 99 -> block 3, row 3
    assert np.array_equal(out[3, 0, :, 3], key[99])
    # rows 4..15 of the partial block and blocks outside the table are untouched
    assert np.array_equal(out[3, :, :, 4:], pool[3, :, :, 4:])
    for b in (0, 4, 6):
        assert np.array_equal(out[b], pool[b])


def test_cache_write_negative_slot_skips_and_others_untouched():
    pool = np.arange(4 * 2 * 2 * 4 * 3, dtype=np.float32).reshape(4, 2, 2, 4, 3)
    key = np.full((3, 2, 3), 7.0, np.float32)
    value = np.full((3, 2, 3), -7.0, np.float32)
    out = oracle.cache_write_ref(pool, key, value, np.array([5, -1, 14]))
    assert np.all(out[1, 0, :, 1] == 7.0) and np.all(out[1, 1, :, 1] == -7.0)   # slot 5
    assert np.all(out[3, 0, :, 2] == 7.0)                                         # slot 14
    changed = np.zeros(pool.shape, bool)
    changed[1, :, :, 1] = changed[3, :, :, 2] = True
    assert np.array_equal(out[~changed], pool[~changed])


def test_cow_copy_happens_before_scatter():
    rng = np.random.default_rng(1)
    pool = rng.standard_normal((6, 2, 2, 8, 4)).astype(np.float16)
    key = rng.standard_normal((1, 2, 4)).astype(np.float16)
    value = rng.standard_normal((1, 2, 4)).astype(np.float16)
    # copy block 2 -> 5, then write one row into block 5 at row 3
    out = oracle.cache_write_ref(pool, key, value, np.array([5 * 8 + 3]), cow_pairs=[(2, 5)])
    expect = pool[2].copy()
    expect[0, :, 3] = key[0]
    expect[1, :, 3] = value[0]
    assert np.array_equal(out[5], expect)
    assert np.array_equal(out[2], pool[2])          # the shared original is intact
    assert np.array_equal(out[:2], pool[:2])


# --------------------------------------------------------------------------
# Block-manager model
# --------------------------------------------------------------------------
def _check_invariants(bm):
    refs = [0] * bm.num_blocks
    for seq, table in bm.tables.items():
        assert len(table) == -(-bm.num_tokens[seq] // bm.block_size)
        for b in table:
            refs[b] += 1
    assert refs == bm.ref_counts                       # every reference is a table entry
    free = set(bm.free_blocks)
    assert len(free) == len(bm.free_blocks)            # no block freed twice
    held = {b for b in range(bm.num_blocks) if refs[b] > 0}
    assert free.isdisjoint(held) and free | held == set(range(bm.num_blocks))
    f, u, s = bm.stats()
    assert (f, u, s) == (len(free), len(held), sum(1 for r in refs if r >= 2))


def test_allocate_takes_ceil_blocks_from_the_stack_end():
    bm = BlockManagerModel(10, 16)
    assert bm.allocate("a", 100) == [9, 8, 7, 6, 5, 4, 3]   # ceil(100/16) = 7 ([KVPA] §4.2)
    assert bm.block_table("a") == ([9, 8, 7, 6, 5, 4, 3], 100)
    # next token (t = 100) goes to row 100 % 16 = 4 of the last block
    assert bm.append_slot("a") == (3 * 16 + 4, -1, -1)
    _check_invariants(bm)


def test_append_at_block_boundary_takes_a_new_block():
    bm = BlockManagerModel(4, 8)
    bm.allocate(1, 8)
    slot, s, d = bm.append_slot(1)        # t = 8: ceil(9/8) = 2 blocks needed
    assert (slot, s, d) == (2 * 8 + 0, -1, -1)
    assert bm.block_table(1) == ([3, 2], 9)


def test_out_of_blocks_leaves_state_unchanged():
    bm = BlockManagerModel(3, 4)
    bm.allocate("a", 12)                  # 3 full blocks; nothing left
    snap = lambda: (list(bm.free_blocks), list(bm.ref_counts), dict(bm.num_tokens),
                    {k: list(v) for k, v in bm.tables.items()})
    before = snap()
    for call in (lambda: bm.allocate("b", 1), lambda: bm.append_slot("a")):
        with pytest.raises(BlockManagerError) as e:
            call()
        assert e.value.kind == "oom"
        assert snap() == before
    # copy-on-write also needs a free block
    bm2 = BlockManagerModel(2, 4)
    bm2.allocate("a", 6)
    bm2.fork("a", "b")
    before2 = (list(bm2.free_blocks), list(bm2.ref_counts))
    with pytest.raises(BlockManagerError):
        bm2.append_slot("b")
    assert (list(bm2.free_blocks), list(bm2.ref_counts)) == before2


def test_unknown_and_double_free_are_errors():
    bm = BlockManagerModel(4, 4)
    bm.allocate(1, 5)
    bm.free(1)
    with pytest.raises(BlockManagerError) as e:
        bm.free(1)
    assert e.value.kind == "not_found"
    assert sorted(bm.free_blocks) == [0, 1, 2, 3] and bm.ref_counts == [0] * 4


def test_fork_then_write_copies_the_shared_partial_block():
    """[NANO] §2.3: B forks from A; the first write into the shared partial block
    gives the writer a private copy and leaves the other sequence on the original."""
    bm = BlockManagerModel(8, 16)
    bm.allocate("A", 30)                  # blocks [7, 6]; block 6 holds 14 rows
    bm.fork("A", "B")
    assert bm.ref_count(7) == 2 and bm.ref_count(6) == 2
    slot, src, dst = bm.append_slot("B")
    assert (src, dst) == (6, 5) and slot == 5 * 16 + 14
    assert bm.block_table("B") == ([7, 5], 31)
    assert bm.block_table("A") == ([7, 6], 30)
    assert bm.ref_count(6) == 1 and bm.ref_count(5) == 1 and bm.ref_count(7) == 2
    # A now owns block 6 alone: no copy
    assert bm.append_slot("A") == (6 * 16 + 14, -1, -1)
    _check_invariants(bm)
    bm.free("A")
    bm.free("B")
    assert sorted(bm.free_blocks) == list(range(8)) and bm.ref_counts == [0] * 8


def test_share_adds_references_and_checks_token_count():
    bm = BlockManagerModel(8, 4)
    prefix = bm.allocate("p", 8)           # two full blocks
    bm.share("x", prefix, 8)
    assert [bm.ref_count(b) for b in prefix] == [2, 2]
    assert bm.block_table("x") == (prefix, 8)
    with pytest.raises(BlockManagerError):
        bm.share("y", prefix, 9)            # 9 tokens need 3 blocks
    with pytest.raises(BlockManagerError):
        bm.share("y", [0], 4)               # block 0 is free
    # a full shared last block needs no copy: the next token opens a new block
    slot, src, dst = bm.append_slot("x")
    assert src == -1 and dst == -1 and slot // 4 not in prefix
    _check_invariants(bm)


OPS = st.lists(st.tuples(st.sampled_from(["alloc", "fork", "append", "free", "share"]),
                         st.integers(0, 5), st.integers(0, 5), st.integers(0, 40)),
               max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops=OPS, bs=st.sampled_from([1, 2, 4, 8]), nb=st.integers(1, 24))
def test_random_lifecycles_keep_invariants_and_free_back_to_initial(ops, bs, nb):
    bm = BlockManagerModel(nb, bs)
    live_slots = {}
    for op, a, b, n in ops:
        try:
            if op == "alloc":
                bm.allocate(a, n)
            elif op == "fork":
                bm.fork(a, b)
            elif op == "append":
                slot, src, dst = bm.append_slot(a)
                table, ntok = bm.block_table(a)
                assert slot // bs == table[-1] and slot % bs == (ntok - 1) % bs
                if src >= 0:
                    assert bm.ref_count(src) >= 1 and bm.ref_count(dst) == 1
            elif op == "free":
                bm.free(a)
            elif op == "share":
                if b in bm.tables and bm.num_tokens[b] % bs == 0:
                    table, ntok = bm.block_table(b)
                    bm.share(a, table, ntok)
        except BlockManagerError:
            pass
        _check_invariants(bm)
        # a block in two tables is a shared block
        owners = {}
        for seq, table in bm.tables.items():
            for blk in table:
                owners.setdefault(blk, set()).add(seq)
        for blk, seqs in owners.items():
            if len(seqs) > 1:
                assert bm.ref_count(blk) >= 2
    for seq in list(bm.tables):
        bm.free(seq)
    assert sorted(bm.free_blocks) == list(range(nb)) and bm.ref_counts == [0] * nb
