"""Pins for the CPU oracle: each test checks the oracle against something other
than itself — values printed on the pages, closed forms, library routines on
contiguous data, exact special cases and invariants.  CPU only."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import kv_size

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Closed forms ([KVPA] §1.2; [KV2P] §2.2, §5.1; [NANO] §1.2)
# --------------------------------------------------------------------------
def test_kv_size_closed_forms_match_page_examples():
    for case in _load("kv_sizes.json")["cases"]:
        got = kv_size.kv_bytes(case["num_layers"], case["kv_width"], case["num_tokens"],
                               case["dtype_bytes"])
        assert got == case["bytes"], case["source"]
        if "values" in case:
            assert kv_size.kv_values_per_token_layer(case["num_kv_heads"], case["head_dim"]) \
                == case["values"]


def test_70b_example_misprint_is_not_the_formula():
    case = _load("kv_sizes.json")["cases"][0]
    assert 80 * 2 * 8192 * 4096 * 2 == case["bytes"] != case["page_printed_bytes"]


def test_blocks_needed_examples():
    ex = _load("paging_example.json")
    assert kv_size.blocks_needed(ex["num_tokens"], ex["block_size"]) == ex["num_blocks"]
    # appending token t needs ceil((t+1)/bs) blocks ([KVPA] §5.3)
    bs = 16
    for t in range(0, 200):
        assert kv_size.blocks_needed(t + 1, bs) == math.ceil((t + 1) / bs)
    assert kv_size.blocks_needed(0, bs) == 0


def test_decode_kv_bytes_is_sum_of_per_token_bytes():
    # 7B MHA (32 heads x 128, fp16): 16 KiB per token per layer
    assert kv_size.decode_kv_bytes([4096] * 32, 32, 128, 2) == 32 * 4096 * 16384
    # 7B GQA (8 KV heads x 128, fp16): 4 KiB per token per layer
    assert kv_size.decode_kv_bytes([100, 1], 8, 128, 2) == 101 * 4096


# --------------------------------------------------------------------------
# Paging example ([KVPA] §4.2)
# --------------------------------------------------------------------------
def _slot_id_pool(num_blocks, block_size, heads=1, head_dim=4):
    """Pool whose every row carries its own (block, row) id in all elements."""
    kv = np.zeros((num_blocks, 2, heads, block_size, head_dim))
    for b in range(num_blocks):
        for r in range(block_size):
            kv[b, 0, :, r, :] = b * 1000 + r
            kv[b, 1, :, r, :] = -(b * 1000 + r)
    return kv


def test_gather_follows_page_paging_example():
    ex = _load("paging_example.json")
    kv = _slot_id_pool(10, ex["block_size"])
    k, v = oracle.gather_sequence(kv, np.array(ex["block_table"]), ex["num_tokens"])
    assert k.shape[0] == ex["num_tokens"]
    for rng in ex["ranges"]:
        lo, hi = rng["tokens"]
        for t in range(lo, hi + 1):
            assert k[t, 0, 0] == rng["physical"] * 1000 + (t - lo)
            assert v[t, 0, 0] == -(rng["physical"] * 1000 + (t - lo))


def test_decode_scale_zero_averages_page_example_rows():
    """scale 0 makes every weight equal: the output is the mean of the V rows the
    page's table maps to.  The expected mean comes from the printed ranges."""
    ex = _load("paging_example.json")
    kv = _slot_id_pool(10, ex["block_size"])
    expected = []
    for rng in ex["ranges"]:
        lo, hi = rng["tokens"]
        expected += [-(rng["physical"] * 1000 + (t - lo)) for t in range(lo, hi + 1)]
    q = np.ones((1, 1, 4))
    out = oracle.decode_ref(q, kv, np.array([ex["block_table"]]), np.array([100]), 0.0)
    assert np.allclose(out[0, 0], np.mean(expected), rtol=0, atol=1e-9)


def test_decode_picks_token_99_from_block_3_row_3():
    """A key that dominates every other picks its own V row: token 99 of the
    page's example lives in physical block 3, row 3."""
    ex = _load("paging_example.json")
    bs = ex["block_size"]
    rng_ = np.random.default_rng(0)
    kv = rng_.standard_normal((10, 2, 1, bs, 4)) * 0.01
    kv[3, 0, 0, 3, :] = [100.0, 0, 0, 0]
    kv[3, 1, 0, 3, :] = [7.0, -7.0, 3.0, 1.0]
    q = np.array([[[1.0, 0, 0, 0]]])
    out = oracle.decode_ref(q, kv, np.array([ex["block_table"]]), np.array([100]), 1.0)
    assert np.allclose(out[0, 0], [7.0, -7.0, 3.0, 1.0], atol=1e-12)
    # with 99 tokens the dominant key is out of range and must not count
    out99 = oracle.decode_ref(q, kv, np.array([ex["block_table"]]), np.array([99]), 1.0)
    assert np.abs(out99[0, 0]).max() < 0.1


# --------------------------------------------------------------------------
# P1: brute force on contiguous K/V with a library attention routine
# --------------------------------------------------------------------------
def _paged_from_contiguous(ks, vs, block_size, num_blocks, seed):
    """Scatter per-sequence contiguous K/V ([n, Hkv, D]) into a random pool."""
    rng_ = np.random.default_rng(seed)
    hkv, d = ks[0].shape[1], ks[0].shape[2]
    pool = rng_.standard_normal((num_blocks, 2, hkv, block_size, d))
    perm = rng_.permutation(num_blocks)
    nbs = [-(-k.shape[0] // block_size) for k in ks]
    tables = np.full((len(ks), max(1, max(nbs))), -1, dtype=np.int64)
    pos = 0
    for s, (k, v) in enumerate(zip(ks, vs)):
        for i in range(nbs[s]):
            b = perm[pos]
            pos += 1
            tables[s, i] = b
            rows = k[i * block_size:(i + 1) * block_size]
            pool[b, 0, :, :rows.shape[0], :] = rows.transpose(1, 0, 2)
            pool[b, 1, :, :rows.shape[0], :] = v[i * block_size:(i + 1) * block_size].transpose(1, 0, 2)
    return pool, tables


@pytest.mark.parametrize("seed,lens,hq,hkv,d,bs", [
    (0, [100, 37, 16, 1], 8, 8, 64, 16),
    (1, [5, 64, 33], 8, 2, 16, 8),
    (2, [31, 1, 70], 4, 1, 32, 32),
    (3, [129, 17], 16, 4, 8, 16),
])
def test_decode_matches_sdpa_on_contiguous_kv(seed, lens, hq, hkv, d, bs):
    rng_ = np.random.default_rng(seed)
    ks = [rng_.standard_normal((n, hkv, d)) for n in lens]
    vs = [rng_.standard_normal((n, hkv, d)) for n in lens]
    q = rng_.standard_normal((len(lens), hq, d))
    num_blocks = sum(-(-n // bs) for n in lens) + 5
    pool, tables = _paged_from_contiguous(ks, vs, bs, num_blocks, seed)
    scale = 1.0 / math.sqrt(d)
    out = oracle.decode_ref(q, pool, tables, np.array(lens), scale)
    for s, n in enumerate(lens):
        kt = torch.from_numpy(ks[s]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        vt = torch.from_numpy(vs[s]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        qt = torch.from_numpy(q[s])[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0, :]
        np.testing.assert_allclose(out[s], ref.numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# P2: physical-permutation invariance (bitwise)
# --------------------------------------------------------------------------
def test_decode_invariant_under_physical_block_permutation():
    x = synth.tiny(seed=4)
    kv = x.kv_cache.numpy()
    bt = x.block_tables.numpy()
    cl = x.context_lens.numpy()
    q = x.q.numpy()
    out = oracle.decode_ref(q, kv, bt, cl, x.scale)
    perm = np.random.default_rng(9).permutation(kv.shape[0])
    kv2 = np.empty_like(kv)
    kv2[perm] = kv                       # block b moves to perm[b]
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    out2 = oracle.decode_ref(q, kv2, bt2, cl, x.scale)
    assert np.array_equal(out, out2)


# --------------------------------------------------------------------------
# P4: special cases
# --------------------------------------------------------------------------
def test_single_token_returns_its_value_row_exactly():
    x = synth.make_decode_inputs([1, 1, 1], 4, 2, 16, 8, dtype="f16", seed=5)
    out = oracle.decode_ref(x.q.numpy(), x.kv_cache.numpy(), x.block_tables.numpy(),
                            x.context_lens.numpy(), x.scale)
    kv = x.kv_cache.numpy()
    for s in range(3):
        b = x.block_tables[s, 0].item()
        for h in range(4):
            assert np.array_equal(out[s, h], kv[b, 1, h // 2, 0].astype(np.float64))


def test_equal_scores_give_mean_of_values():
    x = synth.make_decode_inputs([23, 50], 4, 4, 8, 16, dtype="f32", seed=6)
    out = oracle.decode_ref(x.q.numpy(), x.kv_cache.numpy(), x.block_tables.numpy(),
                            x.context_lens.numpy(), 0.0)
    kv = x.kv_cache.numpy().astype(np.float64)
    for s, n in enumerate([23, 50]):
        rows = [kv[x.block_tables[s, t // 16].item(), 1, :, t % 16, :] for t in range(n)]
        np.testing.assert_allclose(out[s], np.mean(rows, axis=0), rtol=0, atol=1e-12)


def test_output_is_convex_combination_of_values():
    x = synth.make_decode_inputs([77, 3, 128], 8, 2, 32, 16, dtype="f16", seed=7)
    out = oracle.decode_ref(x.q.numpy(), x.kv_cache.numpy(), x.block_tables.numpy(),
                            x.context_lens.numpy(), 3.0)
    kv = x.kv_cache.numpy().astype(np.float64)
    for s, n in enumerate([77, 3, 128]):
        rows = np.stack([kv[x.block_tables[s, t // 16].item(), 1, :, t % 16, :] for t in range(n)])
        for h in range(8):
            lo, hi = rows[:, h // 4].min(0), rows[:, h // 4].max(0)
            assert np.all(out[s, h] >= lo - 1e-12) and np.all(out[s, h] <= hi + 1e-12)


def test_zero_context_gives_zero_output():
    x = synth.make_decode_inputs([0, 5], 2, 2, 8, 8, dtype="f32", seed=8, num_blocks=4)
    out = oracle.decode_ref(x.q.numpy(), x.kv_cache.numpy(), x.block_tables.numpy(),
                            x.context_lens.numpy(), x.scale)
    assert np.all(out[0] == 0) and np.all(np.isfinite(out))


def test_rows_past_context_are_never_read():
    x = synth.tiny(seed=1)
    y = synth.tiny(seed=1, fill_unused=float("nan"))
    args = lambda z: (z.q.numpy(), z.kv_cache.numpy(), z.block_tables.numpy(),
                      z.context_lens.numpy(), z.scale)
    a = oracle.decode_ref(*args(x))
    b = oracle.decode_ref(*args(y))
    assert np.isnan(y.kv_cache.numpy()).any()
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# P5: split-context partials + log-sum-exp merge == single pass
# --------------------------------------------------------------------------
@pytest.mark.parametrize("part", [16, 48, 512])
def test_split_merge_equals_single_pass(part):
    x = synth.make_decode_inputs([700, 1, 16, 513, 0, 35], 8, 2, 32, 16, dtype="f16", seed=10)
    args = (x.q.numpy(), x.kv_cache.numpy(), x.block_tables.numpy(), x.context_lens.numpy(),
            x.scale)
    full = oracle.decode_ref(*args)
    m, l, o = oracle.split_ref(*args, part)
    assert m.shape[2] == -(-700 // part)
    merged = oracle.merge_ref(m, l, o)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-12)


def test_partials_are_attention_over_their_token_range():
    """A partition's normalised output is attention restricted to its tokens:
    compare with SDPA on the contiguous slice."""
    x = synth.make_decode_inputs([300], 2, 1, 16, 16, dtype="f32", seed=11)
    args = (x.q.numpy(), x.kv_cache.numpy(), x.block_tables.numpy(), x.context_lens.numpy(),
            x.scale)
    m, l, o = oracle.split_ref(*args, 128)
    k, v = oracle.gather_sequence(x.kv_cache.numpy(), x.block_tables.numpy()[0], 300)
    for p, (lo, hi) in enumerate([(0, 128), (128, 256), (256, 300)]):
        kt = torch.from_numpy(k[lo:hi, 0].astype(np.float64))[None].expand(2, -1, -1)
        vt = torch.from_numpy(v[lo:hi, 0].astype(np.float64))[None].expand(2, -1, -1)
        qt = torch.from_numpy(x.q.numpy()[0].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=x.scale)[:, 0]
        np.testing.assert_allclose(o[0, :, p], ref.numpy(), rtol=0, atol=1e-12)
        z = x.scale * (k[lo:hi, 0].astype(np.float64) @ x.q.numpy()[0].astype(np.float64).T)
        np.testing.assert_allclose(m[0, :, p], z.max(0), rtol=0, atol=1e-12)
        np.testing.assert_allclose(l[0, :, p], np.exp(z - z.max(0)).sum(0), rtol=1e-12)


def test_merge_of_one_partition_is_identity_and_empty_is_zero():
    o = np.random.default_rng(0).standard_normal((2, 3, 1, 8))
    m = np.zeros((2, 3, 1))
    l = np.ones((2, 3, 1)) * 2.5
    assert np.allclose(oracle.merge_ref(m, l, o), o[:, :, 0], atol=1e-15)
    l[1, 2, 0] = 0
    m[1, 2, 0] = -np.inf
    assert np.all(oracle.merge_ref(m, l, o)[1, 2] == 0)


# --------------------------------------------------------------------------
# sliding window ([KV2P] §7.2)
# --------------------------------------------------------------------------
from tests import pins as _pins


@pytest.mark.parametrize("window", [1, 7, 16, 33, 64, 1000])
def test_window_equals_sdpa_on_last_tokens(window):
    assert _pins.window_is_sdpa_on_last_tokens(oracle.decode_ref, window)


def test_window_one_returns_newest_value_row():
    assert _pins.window_one_is_last_value(oracle.decode_ref)


def test_window_larger_than_context_is_full_attention():
    x = synth.make_decode_inputs([20, 300], 4, 2, 16, 16, dtype="f32", seed=23)
    args = (x.q.numpy(), x.kv_cache.numpy(), x.block_tables.numpy(), x.context_lens.numpy(),
            x.scale)
    assert np.array_equal(oracle.decode_ref(*args, window=300), oracle.decode_ref(*args))
    assert not np.allclose(oracle.decode_ref(*args, window=299), oracle.decode_ref(*args))


# --------------------------------------------------------------------------
# multi-token queries with a causal mask ([KV2P] §5.4; [INFRA] §2)
# --------------------------------------------------------------------------
def test_prefill_is_end_aligned_causal_sdpa():
    assert _pins.prefill_is_masked_sdpa(oracle.prefill_ref)


def test_prefill_single_token_is_decode():
    assert _pins.prefill_single_token_is_decode(oracle.prefill_ref, oracle.decode_ref)


def test_prefill_in_chunks_equals_at_once():
    assert _pins.chunked_equals_whole(oracle.prefill_ref)


def test_prefill_first_query_of_fresh_prompt_is_its_value_row():
    """n = T: query 0 sees only key 0, whose V row it returns."""
    rng = np.random.default_rng(14)
    kv = rng.standard_normal((4, 2, 1, 8, 8))
    q = rng.standard_normal((5, 2, 8))
    out = oracle.prefill_ref(q, kv, np.array([[2, 0]]), np.array([5]), np.array([0, 5]), 1.0)
    assert np.array_equal(out[0, 0], kv[2, 1, 0, 0]) and np.array_equal(out[0, 1], kv[2, 1, 0, 0])


# sliding window on multi-token queries ([KV2P] §7.2 applied per query)
@pytest.mark.parametrize("window", [1, 3, 16, 39, 100])
def test_prefill_window_is_banded_sdpa(window):
    assert _pins.prefill_window_is_banded_sdpa(oracle.prefill_ref, window)


def test_prefill_window_one_is_own_value_row():
    assert _pins.prefill_window_one_is_own_value_row(oracle.prefill_ref)


def test_prefill_window_single_token_is_windowed_decode():
    """T = 1 per sequence under a window is the windowed decode, exactly."""
    rng = np.random.default_rng(16)
    kv = rng.standard_normal((12, 2, 2, 8, 16))
    bt = np.array([[3, 1, 7], [4, 0, 11]])
    lens = np.array([20, 9])
    q = rng.standard_normal((2, 4, 16))
    for w in (1, 5, 9, 19, 50):
        assert np.array_equal(oracle.prefill_ref(q, kv, bt, lens, np.array([0, 1, 2]), 0.5,
                                                 window=w),
                              oracle.decode_ref(q, kv, bt, lens, 0.5, window=w))


def test_prefill_window_at_least_context_is_plain_causal():
    rng = np.random.default_rng(17)
    kv = rng.standard_normal((10, 2, 2, 8, 16))
    bt = np.array([[3, 1, 7, 9], [4, 0, 2, 5]])
    lens, qs = np.array([30, 12]), np.array([0, 10, 22])
    q = rng.standard_normal((22, 4, 16))
    full = oracle.prefill_ref(q, kv, bt, lens, qs, 0.4)
    assert np.array_equal(oracle.prefill_ref(q, kv, bt, lens, qs, 0.4, window=30), full)
    assert not np.allclose(oracle.prefill_ref(q, kv, bt, lens, qs, 0.4, window=29), full)
