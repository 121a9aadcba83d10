"""Pins for the block manager's prefix cache ([KVPA] §8.1-§8.2; [KV2P]
§4.2-§4.3; [NANO] §3.2, §4.3): the FNV-1a primitive against its published test
values, scenarios the pages describe (one copy of a shared system prompt,
block-level matching that depends on position, multi-turn reuse of full
blocks, LRU eviction that spares referenced blocks, protection of hot
prefixes) and the bookkeeping invariants over random lifecycles.  CPU only."""

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import BlockManagerError, BlockManagerModel
from oracle.block_manager import fnv1a64
from tests import pins


def test_fnv1a64_published_values():
    assert pins.fnv_vectors(fnv1a64)


def test_system_prompt_stored_once():
    assert pins.system_prompt_stored_once(BlockManagerModel)


def test_block_hash_depends_on_position():
    assert pins.position_matters(BlockManagerModel)


def test_multi_turn_reuses_full_blocks_only():
    assert pins.multi_turn_reuses_full_blocks(BlockManagerModel)


def test_lru_eviction_spares_referenced_blocks():
    assert pins.lru_spares_referenced_blocks(BlockManagerModel)


def test_protection_keeps_hot_prefix():
    assert pins.protection_keeps_hot_prefix(BlockManagerModel)


def test_admission_threshold_keeps_one_shot_prompts_out():
    assert pins.admission_threshold_keeps_one_shot_prompts_out(BlockManagerModel)


def test_admission_table_is_bounded():
    assert pins.admission_table_is_bounded(BlockManagerModel)


def test_prefix_cache_needs_empty_manager_and_is_off_by_default():
    m = BlockManagerModel(8, 4)
    try:
        m.allocate_prompt(0, [1, 2, 3, 4])
        raise AssertionError("allocate_prompt with the cache off must fail")
    except BlockManagerError as e:
        assert e.kind == "invalid"
    m.allocate(1, 4)
    try:
        m.enable_prefix_cache()
        raise AssertionError
    except BlockManagerError as e:
        assert e.kind == "invalid"


def test_oom_leaves_state_unchanged():
    m = BlockManagerModel(4, 4)
    m.enable_prefix_cache()
    m.allocate_prompt(0, list(range(8)))
    m.register(0)
    before = (list(m.free_blocks), list(m.ref_counts), dict(m.evictable), m.prefix_stats())
    try:
        m.allocate_prompt(1, list(range(8)) + list(range(100, 112)))   # 2 hits + 3 fresh > 2
        raise AssertionError
    except BlockManagerError as e:
        assert e.kind == "oom"
    assert (list(m.free_blocks), list(m.ref_counts), dict(m.evictable), m.prefix_stats()) == before


def test_record_tokens_then_register_caches_decoded_blocks():
    m = BlockManagerModel(16, 4)
    m.enable_prefix_cache()
    m.allocate_prompt(0, [1, 2, 3, 4, 5, 6])
    assert m.register(0) == 1
    for t in (7, 8, 9):
        m.append_slot(0)
    m.record_tokens(0, [7, 8, 9])
    assert m.register(0) == 1                     # tokens 5..8 fill block 1
    m.free(0)
    _, cached = m.allocate_prompt(1, [1, 2, 3, 4, 5, 6, 7, 8, 9])
    assert cached == 8


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 5), st.integers(0, 7), st.integers(0, 40)),
                min_size=1, max_size=40), st.integers(0, 3))
def test_invariants_over_random_lifecycles(ops, protect):
    m = BlockManagerModel(24, 4)
    m.enable_prefix_cache(protect_hits=protect)
    prompts = [list(np.random.default_rng(k).integers(0, 3, 40)) for k in range(4)]
    live = set()
    for op, a, n in ops:
        try:
            if op <= 1:
                if a not in live:
                    m.allocate_prompt(a, prompts[a % 4][:n])
                    live.add(a)
            elif op == 2 and a in live:
                m.register(a)
            elif op == 3 and a in live:
                m.append_slot(a)
            elif op == 4 and a in live:
                m.free(a)
                live.discard(a)
            elif op == 5 and a in live and (a + 1) not in live:
                m.fork(a, a + 1)
                live.add(a + 1)
        except BlockManagerError as e:
            assert e.kind == "oom"
        assert pins.prefix_invariants(m)
        assert pins.invariants_hold(m)
    for s in list(live):
        m.free(s)
    assert pins.prefix_invariants(m) and m.stats()[1] == 0
