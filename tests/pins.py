"""Pin checks for a decode-attention implementation, shared by the oracle's
pin tests and the mutation tests that show the pins catch plausible
mistakes.  Each check returns True when `decode` agrees with something other
than itself: values printed on the pages, a library routine on contiguous
data, exact special cases or invariants.  CPU only."""

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def page_example():
    with open(os.path.join(GOLDEN, "paging_example.json")) as f:
        return json.load(f)


def _slot_id_pool(num_blocks, block_size, heads=1, head_dim=4):
    kv = np.zeros((num_blocks, 2, heads, block_size, head_dim))
    for b in range(num_blocks):
        for r in range(block_size):
            kv[b, 0, :, r, :] = b * 1000 + r
            kv[b, 1, :, r, :] = -(b * 1000 + r)
    return kv


def scale_zero_page_example(decode):
    """scale 0: the mean of the V rows the page's table maps (printed ranges)."""
    ex = page_example()
    kv = _slot_id_pool(10, ex["block_size"])
    expect = []
    for rng in ex["ranges"]:
        lo, hi = rng["tokens"]
        expect += [-(rng["physical"] * 1000 + (t - lo)) for t in range(lo, hi + 1)]
    out = decode(np.ones((1, 1, 4)), kv, np.array([ex["block_table"]]), np.array([100]), 0.0)
    return bool(np.allclose(out[0, 0], np.mean(expect), rtol=0, atol=1e-9))


def dominant_key_token_99(decode):
    """A dominant key at token 99 (block 3, row 3 on the page) picks its V row;
    with 99 tokens it must not count."""
    ex = page_example()
    bs = ex["block_size"]
    kv = np.random.default_rng(0).standard_normal((10, 2, 1, bs, 4)) * 0.01
    kv[3, 0, 0, 3, :] = [100.0, 0, 0, 0]
    kv[3, 1, 0, 3, :] = [7.0, -7.0, 3.0, 1.0]
    q = np.array([[[1.0, 0, 0, 0]]])
    a = decode(q, kv, np.array([ex["block_table"]]), np.array([100]), 1.0)
    b = decode(q, kv, np.array([ex["block_table"]]), np.array([99]), 1.0)
    return bool(np.allclose(a[0, 0], [7.0, -7.0, 3.0, 1.0], atol=1e-9)
                and np.abs(b[0, 0]).max() < 0.1)


def sdpa_on_contiguous(decode, seed=1, lens=(5, 64, 33), hq=8, hkv=2, d=16, bs=8):
    """Agreement with torch SDPA on contiguous K/V scattered into a random pool."""
    rng = np.random.default_rng(seed)
    ks = [rng.standard_normal((n, hkv, d)) for n in lens]
    vs = [rng.standard_normal((n, hkv, d)) for n in lens]
    q = rng.standard_normal((len(lens), hq, d))
    nbs = [-(-n // bs) for n in lens]
    nb = sum(nbs) + 5
    pool = rng.standard_normal((nb, 2, hkv, bs, d))
    perm = rng.permutation(nb)
    tables = np.full((len(lens), max(nbs)), -1, dtype=np.int64)
    pos = 0
    for s, (k, v) in enumerate(zip(ks, vs)):
        for i in range(nbs[s]):
            b = perm[pos]
            pos += 1
            tables[s, i] = b
            rows = k[i * bs:(i + 1) * bs]
            pool[b, 0, :, :rows.shape[0], :] = rows.transpose(1, 0, 2)
            pool[b, 1, :, :rows.shape[0], :] = v[i * bs:(i + 1) * bs].transpose(1, 0, 2)
    scale = 1.0 / math.sqrt(d)
    out = decode(q, pool, tables, np.array(lens), scale)
    for s in range(len(lens)):
        kt = torch.from_numpy(ks[s]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        vt = torch.from_numpy(vs[s]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[s])[:, None, :], kt, vt, scale=scale)[:, 0, :]
        if not np.allclose(out[s], ref.numpy(), rtol=0, atol=1e-12):
            return False
    return True


def single_token_exact(decode):
    """n = 1 returns the V row exactly."""
    rng = np.random.default_rng(5)
    kv = rng.standard_normal((4, 2, 2, 8, 16))
    q = rng.standard_normal((2, 4, 16))
    bt = np.array([[2], [0]])
    out = decode(q, kv, bt, np.array([1, 1]), 0.25)
    return bool(np.array_equal(out[0, 3], kv[2, 1, 1, 0]) and np.array_equal(out[1, 0], kv[0, 1, 0, 0]))


def rows_past_context_ignored(decode):
    """NaN in every row no context covers changes nothing."""
    rng = np.random.default_rng(6)
    kv = rng.standard_normal((6, 2, 2, 8, 16))
    q = rng.standard_normal((2, 2, 16))
    bt = np.array([[4, 1], [3, -1]])
    lens = np.array([11, 3])
    a = decode(q, kv, bt, lens, 0.3)
    kv2 = kv.copy()
    kv2[4, :, :, :, :] = kv[4]
    kv2[1, :, :, 3:, :] = np.nan
    kv2[3, :, :, 3:, :] = np.nan
    kv2[[0, 2, 5]] = np.nan
    b = decode(q, kv2, bt, lens, 0.3)
    return bool(np.array_equal(a, b))


ALL = [scale_zero_page_example, dominant_key_token_99, sdpa_on_contiguous, single_token_exact,
       rows_past_context_ignored]


def failing(decode):
    """Names of the pins `decode` fails (an exception counts as a failure)."""
    bad = []
    for pin in ALL:
        try:
            ok = pin(decode)
        except Exception:
            ok = False
        if not ok:
            bad.append(pin.__name__)
    return bad


# --------------------------------------------------------------------------
# cache write pins
# --------------------------------------------------------------------------
def cache_round_trip(cache_write, gather):
    """Rows written at the slots of the page's printed ranges read back, in
    order, through the page's table; untouched rows stay."""
    ex = page_example()
    bs, n = ex["block_size"], ex["num_tokens"]
    rng = np.random.default_rng(0)
    pool = rng.standard_normal((10, 2, 3, bs, 8)).astype(np.float16)
    key = rng.standard_normal((n, 3, 8)).astype(np.float16)
    value = rng.standard_normal((n, 3, 8)).astype(np.float16)
    slots = np.empty(n, dtype=np.int64)
    for r in ex["ranges"]:
        lo, hi = r["tokens"]
        slots[lo:hi + 1] = r["physical"] * bs + np.arange(hi - lo + 1)
    out = cache_write(pool, key, value, slots)
    k, v = gather(out, np.array(ex["block_table"]), n)
    return bool(np.array_equal(k, key) and np.array_equal(v, value)
                and np.array_equal(out[3, :, :, 4:], pool[3, :, :, 4:])
                and np.array_equal(out[0], pool[0]))


def cow_before_scatter(cache_write):
    rng = np.random.default_rng(1)
    pool = rng.standard_normal((6, 2, 2, 8, 4)).astype(np.float16)
    key = rng.standard_normal((1, 2, 4)).astype(np.float16)
    value = rng.standard_normal((1, 2, 4)).astype(np.float16)
    out = cache_write(pool, key, value, np.array([5 * 8 + 3]), cow_pairs=[(2, 5)])
    expect = pool[2].copy()
    expect[0, :, 3] = key[0]
    expect[1, :, 3] = value[0]
    return bool(np.array_equal(out[5], expect) and np.array_equal(out[2], pool[2]))


# --------------------------------------------------------------------------
# block-manager pins
# --------------------------------------------------------------------------
def invariants_hold(bm):
    refs = [0] * bm.num_blocks
    for seq, table in bm.tables.items():
        if len(table) != -(-bm.num_tokens[seq] // bm.block_size):
            return False
        for b in table:
            refs[b] += 1
    free = set(bm.free_blocks)
    held = {b for b in range(bm.num_blocks) if refs[b] > 0}
    idle = set(getattr(bm, "evictable", ()))   # cached, unreferenced (prefix cache)
    return (refs == list(bm.ref_counts) and len(free) == len(bm.free_blocks)
            and free.isdisjoint(held) and idle.isdisjoint(held) and free.isdisjoint(idle)
            and free | held | idle == set(range(bm.num_blocks)))


def bm_fork_cow_example(model_cls):
    """B forks from A (30 tokens, block 16); B's first write copies the shared
    partial block, A keeps the original; freeing both restores the pool."""
    bm = model_cls(8, 16)
    bm.allocate("A", 30)
    bm.fork("A", "B")
    slot, src, dst = bm.append_slot("B")
    ok = (src, dst) == (6, 5) and slot == 5 * 16 + 14 and bm.block_table("A") == ([7, 6], 30)
    ok = ok and bm.append_slot("A") == (6 * 16 + 14, -1, -1) and invariants_hold(bm)
    bm.free("A")
    bm.free("B")
    return bool(ok and sorted(bm.free_blocks) == list(range(8)) and list(bm.ref_counts) == [0] * 8)


def bm_scripted_lifecycle(model_cls):
    """A fixed lifecycle (allocate, share, fork, appends across block
    boundaries and copies, frees) keeps every invariant after every step."""
    bm = model_cls(12, 4)
    steps = [lambda: bm.allocate(0, 6), lambda: bm.share(1, bm.block_table(0)[0][:1], 4),
             lambda: bm.fork(0, 2), lambda: bm.append_slot(2), lambda: bm.append_slot(0),
             lambda: bm.append_slot(1), lambda: bm.append_slot(2), lambda: bm.append_slot(2),
             lambda: bm.free(0), lambda: bm.append_slot(1), lambda: bm.free(2),
             lambda: bm.free(1)]
    for st in steps:
        st()
        if not invariants_hold(bm):
            return False
    return sorted(bm.free_blocks) == list(range(12))


# --------------------------------------------------------------------------
# sliding-window pins
# --------------------------------------------------------------------------
def window_is_sdpa_on_last_tokens(decode, window):
    """With a window W, attention over the last W tokens only: SDPA on the
    contiguous slice [n - W, n) of each sequence (whole context when n <= W)."""
    rng = np.random.default_rng(21)
    lens, hq, hkv, d, bs = (37, 5, 64, 100), 8, 2, 16, 8
    ks = [rng.standard_normal((n, hkv, d)) for n in lens]
    vs = [rng.standard_normal((n, hkv, d)) for n in lens]
    q = rng.standard_normal((len(lens), hq, d))
    nbs = [-(-n // bs) for n in lens]
    pool = rng.standard_normal((sum(nbs) + 3, 2, hkv, bs, d))
    tables = np.full((len(lens), max(nbs)), -1, dtype=np.int64)
    perm = rng.permutation(pool.shape[0])
    pos = 0
    for s, (k, v) in enumerate(zip(ks, vs)):
        for i in range(nbs[s]):
            b = perm[pos]
            pos += 1
            tables[s, i] = b
            r = k[i * bs:(i + 1) * bs]
            pool[b, 0, :, :r.shape[0]] = r.transpose(1, 0, 2)
            pool[b, 1, :, :r.shape[0]] = v[i * bs:(i + 1) * bs].transpose(1, 0, 2)
    scale = 0.25
    out = decode(q, pool, tables, np.array(lens), scale, window=window)
    for s, n in enumerate(lens):
        lo = max(0, n - window)
        kt = torch.from_numpy(ks[s][lo:]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        vt = torch.from_numpy(vs[s][lo:]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[s])[:, None, :], kt, vt, scale=scale)[:, 0, :]
        if not np.allclose(out[s], ref.numpy(), rtol=0, atol=1e-12):
            return False
    return True


def window_one_is_last_value(decode):
    """W = 1: each head returns the V row of the newest token exactly."""
    rng = np.random.default_rng(22)
    kv = rng.standard_normal((5, 2, 2, 8, 16))
    q = rng.standard_normal((2, 4, 16))
    bt = np.array([[3, 1], [4, 0]])
    out = decode(q, kv, bt, np.array([12, 8]), 0.5, window=1)
    return bool(np.array_equal(out[0, 2], kv[1, 1, 1, 3]) and np.array_equal(out[1, 0], kv[4, 1, 0, 7]))


# --------------------------------------------------------------------------
# INT8 group-wise quantisation pins ([KV2P] §5.2)
# --------------------------------------------------------------------------
def quant_integers_exact(quantize):
    """A row of integers whose largest magnitude is 127 has scale exactly 1,
    so its codes are the integers themselves."""
    row = np.array([127, -3, 0, 45, -127, 1, 99, -64], dtype=np.float16)
    codes, scales = quantize(row[None])
    return bool(scales[0] == np.float32(1.0) and np.array_equal(codes[0], row.astype(np.int8)))


def quant_rounds_half_to_even(quantize):
    """At scale 1 the ties x.5 go to the even neighbour."""
    row = np.array([127, 2.5, -2.5, 3.5, 0.5, -0.5, 1.5, -1.5], dtype=np.float16)
    codes, _ = quantize(row[None])
    return bool(np.array_equal(codes[0], np.array([127, 2, -2, 4, 0, 0, 2, -2], dtype=np.int8)))


def quant_scale_is_amax_over_127(quantize):
    """scale * 127 equals the row's largest magnitude to float32 rounding, and
    that element's code is +-127; a zero row has scale 0 and codes 0."""
    rng = np.random.default_rng(5)
    rows = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 50, (64, 1))).astype(np.float16)
    rows[7] = 0
    codes, scales = quantize(rows)
    amax = np.abs(rows.astype(np.float64)).max(axis=1)
    ok = np.all(np.abs(scales.astype(np.float64) * 127 - amax) <= amax * 2.0 ** -22)
    arg = np.abs(rows.astype(np.float64)).argmax(axis=1)
    live = amax > 0
    ok &= np.all(np.abs(codes[np.arange(64), arg][live].astype(int)) == 127)
    ok &= scales[7] == 0 and not codes[7].any()
    return bool(ok)


def quant_error_within_half_step(quantize, dequantize):
    """Every dequantised value is within half a step of its input, and the
    steps are per row: an outlier in one row leaves the others' steps alone."""
    rng = np.random.default_rng(6)
    rows = rng.standard_normal((32, 64)).astype(np.float16)
    rows[3, 10] = 900.0
    codes, scales = quantize(rows)
    back = dequantize(codes, scales)
    err = np.abs(back - rows.astype(np.float64))
    bound = scales.astype(np.float64)[:, None] * (0.5 + 2.0 ** -20)
    amax = np.abs(rows.astype(np.float64)).max(axis=1)
    return bool(np.all(err <= bound) and np.all(scales[np.arange(32) != 3] < 0.05)
                and abs(scales[3] * 127 - 900) < 1e-3
                and np.all(np.abs(back) <= amax[:, None] * (1 + 2.0 ** -22)))


QUANT_PINS = [quant_integers_exact, quant_rounds_half_to_even, quant_scale_is_amax_over_127]


def quant_failing(quantize, dequantize):
    bad = [p.__name__ for p in QUANT_PINS if not p(quantize)]
    if not quant_error_within_half_step(quantize, dequantize):
        bad.append("quant_error_within_half_step")
    return bad


def i8_cache_round_trip(cache_write_i8, quantize, dequantize):
    """Rows written at the slots of the page's printed ranges come back, through
    the page's table, as their own quantisation (codes in [block, K|V, head,
    row], per-row scales in [block, head, K|V, row]); untouched rows and
    scales stay."""
    ex = page_example()
    bs, n = ex["block_size"], ex["num_tokens"]
    rng = np.random.default_rng(2)
    hkv, d = 3, 16
    codes = rng.integers(-127, 128, (10, 2, hkv, bs, d)).astype(np.int8)
    scales = rng.uniform(0.1, 1, (10, hkv, 2, bs)).astype(np.float32)
    key = (rng.standard_normal((n, hkv, d)) * 3).astype(np.float16)
    value = rng.standard_normal((n, hkv, d)).astype(np.float16)
    slots = np.empty(n, dtype=np.int64)
    for r in ex["ranges"]:
        lo, hi = r["tokens"]
        slots[lo:hi + 1] = r["physical"] * bs + np.arange(hi - lo + 1)
    c2, s2 = cache_write_i8(codes, scales, key, value, slots)
    kq, ks = quantize(key)
    vq, vs = quantize(value)
    table = ex["block_table"]
    ok = True
    for t in range(n):
        b, r = table[t // bs], t % bs
        ok &= np.array_equal(c2[b, 0, :, r], kq[t]) and np.array_equal(c2[b, 1, :, r], vq[t])
        ok &= np.array_equal(s2[b, :, 0, r], ks[t]) and np.array_equal(s2[b, :, 1, r], vs[t])
    # block 3 holds tokens 96..99 in rows 0..3 only; blocks 0 and 4 are not in the table
    ok &= np.array_equal(c2[3, :, :, 4:], codes[3, :, :, 4:])
    ok &= np.array_equal(s2[3, :, :, 4:], scales[3, :, :, 4:])
    ok &= np.array_equal(c2[0], codes[0]) and np.array_equal(s2[4], scales[4])
    # dequantised keys are within half a step of the written ones
    back = dequantize(c2[table[0], 0, :, :16].transpose(1, 0, 2), s2[table[0], :, 0, :16].T)
    ok &= np.all(np.abs(back - key[:16].astype(np.float64)) <= ks[:16, :, None] * 0.5001)
    return bool(ok)


def i8_cow_before_scatter(cache_write_i8):
    """Copies go first and carry codes and scales; the source stays intact."""
    rng = np.random.default_rng(3)
    codes = rng.integers(-127, 128, (4, 2, 2, 8, 16)).astype(np.int8)
    scales = rng.uniform(0.1, 1, (4, 2, 2, 8)).astype(np.float32)   # [NB, Hkv, K|V, bs]
    key = np.full((1, 2, 16), 2.0, dtype=np.float16)
    value = np.full((1, 2, 16), -4.0, dtype=np.float16)
    c2, s2 = cache_write_i8(codes, scales, key, value, np.array([2 * 8 + 5]), [(1, 2)])
    ok = np.array_equal(c2[1], codes[1]) and np.array_equal(s2[1], scales[1])
    ok &= np.array_equal(np.delete(c2[2], 5, axis=2), np.delete(codes[1], 5, axis=2))
    ok &= np.array_equal(np.delete(s2[2], 5, axis=2), np.delete(scales[1], 5, axis=2))
    ok &= np.all(c2[2, 0, :, 5] == 127) and np.all(c2[2, 1, :, 5] == -127)
    ok &= np.allclose(s2[2, :, 0, 5], 2 / 127) and np.allclose(s2[2, :, 1, 5], 4 / 127)
    return bool(ok)


def i8_decode_is_sdpa_on_dequantised(decode_i8, dequantize):
    """Decode over the INT8 pool equals SDPA over the dequantised contiguous
    K/V of each sequence (scattered through a random table)."""
    rng = np.random.default_rng(8)
    lens, hq, hkv, d, bs = (40, 3, 17), 8, 2, 16, 8
    nbs = [-(-n // bs) for n in lens]
    nb = sum(nbs) + 2
    codes = rng.integers(-127, 128, (nb, 2, hkv, bs, d)).astype(np.int8)
    scales = rng.uniform(0.001, 0.05, (nb, hkv, 2, bs)).astype(np.float32)
    perm = rng.permutation(nb)
    tables = np.full((len(lens), max(nbs)), -1)
    pos = 0
    for s, k in enumerate(nbs):
        tables[s, :k] = perm[pos:pos + k]
        pos += k
    q = rng.standard_normal((len(lens), hq, d))
    out = decode_i8(q, codes, scales, tables, np.array(lens), 0.3)
    for s, n in enumerate(lens):
        t = np.arange(n)
        blk = tables[s][t // bs]
        kk = codes[blk, 0, :, t % bs, :].astype(np.float64) * scales[blk, :, 0, t % bs][..., None]
        vv = codes[blk, 1, :, t % bs, :].astype(np.float64) * scales[blk, :, 1, t % bs][..., None]
        kt = torch.from_numpy(kk).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        vt = torch.from_numpy(vv).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[s])[:, None, :], kt, vt, scale=0.3)[:, 0, :]
        if not np.allclose(out[s], ref.numpy(), rtol=0, atol=1e-12):
            return False
    return True


# --------------------------------------------------------------------------
# prefix-cache pins ([KVPA] §8.1-§8.2; [KV2P] §4.2-§4.3; [NANO] §3.2, §4.3)
# --------------------------------------------------------------------------
def fnv_vectors(fnv):
    """Published FNV-1a 64-bit test values."""
    return (fnv(b"") == 0xCBF29CE484222325 and fnv(b"a") == 0xAF63DC4C8601EC8C
            and fnv(b"foobar") == 0x85944171F73967E8)


def _toks(seed, n, lo=0, hi=32000):
    return np.random.default_rng(seed).integers(lo, hi, n).tolist()


def system_prompt_stored_once(model_cls):
    """100 requests with the same 512-token system prompt keep one copy of its
    32 blocks: every request after the first reuses all of them."""
    bs, sys_prompt = 16, _toks(1, 512)
    m = model_cls(4096, bs)
    m.enable_prefix_cache()
    got = []
    for r in range(100):
        table, cached = m.allocate_prompt(r, sys_prompt + _toks(100 + r, 20))
        m.register(r)
        got.append((table, cached))
    shared = got[0][0][:32]
    ok = got[0][1] == 0 and all(c == 512 and t[:32] == shared for t, c in got[1:])
    ok &= all(m.ref_count(b) == 100 for b in shared)
    ok &= m.stats()[1] == 32 + 100 * 2
    return bool(ok)


def position_matters(model_cls):
    """A block's hash covers its position: the same 16 tokens after a
    different prefix do not match."""
    bs = 16
    a, b, c = _toks(2, 16), _toks(3, 16), _toks(4, 16)
    m = model_cls(64, bs)
    m.enable_prefix_cache()
    m.allocate_prompt(0, a + b)
    m.register(0)
    _, c1 = m.allocate_prompt(1, b + a)
    _, c2 = m.allocate_prompt(2, a + c)
    _, c3 = m.allocate_prompt(3, c + b)
    _, c4 = m.allocate_prompt(4, a + b + c)
    return (c1, c2, c3, c4) == (0, 16, 0, 32)


def multi_turn_reuses_full_blocks(model_cls):
    """Turn 2 repeats turn 1 and extends it: the full blocks of turn 1 are
    reused, its partial last block is not."""
    bs = 16
    t1 = _toks(5, 40)                      # 2 full blocks + 8 tokens
    m = model_cls(64, bs)
    m.enable_prefix_cache()
    table1, c1 = m.allocate_prompt(0, t1)
    n_reg = m.register(0)
    m.free(0)
    table2, c2 = m.allocate_prompt(1, t1 + _toks(6, 50))
    # (the freed partial block may come back as a fresh block: ids are policy)
    return c1 == 0 and n_reg == 2 and c2 == 32 and table2[:2] == table1[:2] \
        and m.prefix_stats()[3] == 2


def lru_spares_referenced_blocks(model_cls):
    """Eviction takes the least recently released cached block and never one
    that a live sequence holds."""
    bs = 4
    A, B, C = _toks(7, 8), _toks(8, 8), _toks(9, 8)
    m = model_cls(8, bs)
    m.enable_prefix_cache()
    m.allocate_prompt("A", A)
    m.register("A")                        # A stays alive
    for s, t in (("B", B), ("C", C)):
        m.allocate_prompt(s, t)
        m.register(s)
    m.free("B")                            # released first
    m.free("C")
    m.allocate("big", 10)                  # 3 blocks: 2 free + 1 evicted
    evicted_first_b = m.prefix_stats()[5] == 1
    _, cc = m.allocate_prompt("C2", C)     # C and A still match whole
    _, ca = m.allocate_prompt("A2", A)
    m.free("big")
    _, cb = m.allocate_prompt("B2", B)     # B lost its first block: no match
    return bool(evicted_first_b and cb == 0 and cc == 8 and ca == 8)


def protection_keeps_hot_prefix(model_cls):
    """With protect_hits = 2 a block hit twice outlives a once-hit block that
    was released later (plain LRU would evict the hot one first)."""
    bs = 4
    hot, cold = _toks(10, 4), _toks(11, 4)
    m = model_cls(4, bs)
    m.enable_prefix_cache(protect_hits=2)
    for s in ("h0", "h1", "h2"):          # hot block: cached, then hit twice
        m.allocate_prompt(s, hot)
        m.register(s)
    m.allocate_prompt("c0", cold)
    m.register("c0")
    m.allocate_prompt("c1", cold)          # cold: one hit
    for s in ("h0", "h1", "h2"):
        m.free(s)                          # hot released first
    m.free("c0")
    m.free("c1")
    m.allocate("big", 12)                  # 3 blocks: 2 free + 1 evicted
    _, ch = m.allocate_prompt("h3", hot)
    m.free("big")
    _, cc = m.allocate_prompt("c2", cold)
    return ch == 4 and cc == 0


def prefix_invariants(m):
    """Cache bookkeeping: evictable = cached with count 0, free blocks are not
    cached, free + evictable + held partition the pool, the hash map and the
    per-block keys agree."""
    n = m.num_blocks
    held = {b for b in range(n) if m.ref_counts[b] > 0}
    free = set(m.free_blocks)
    ev = set(m.evictable)
    cached = set(m.block_key)
    ok = ev == {b for b in cached if m.ref_counts[b] == 0}
    ok &= not (free & cached) and len(free) == len(m.free_blocks)
    ok &= (free | ev | held) == set(range(n)) and not (free & held) and not (ev & held)
    ok &= all(m.cache[k[0]] == b for b, k in m.block_key.items()) and len(m.cache) == len(cached)
    return bool(ok)


# --------------------------------------------------------------------------
# multi-token (chunked prefill) pins ([KV2P] §5.4; [INFRA] §2)
# --------------------------------------------------------------------------
def _scatter(ks, vs, bs, seed):
    rng = np.random.default_rng(seed)
    hkv, d = ks[0].shape[1], ks[0].shape[2]
    nbs = [-(-k.shape[0] // bs) for k in ks]
    nb = sum(nbs) + 3
    pool = rng.standard_normal((nb, 2, hkv, bs, d))
    perm = rng.permutation(nb)
    tables = np.full((len(ks), max(nbs)), -1, dtype=np.int64)
    pos = 0
    for s, (k, v) in enumerate(zip(ks, vs)):
        for i in range(nbs[s]):
            b = perm[pos]
            pos += 1
            tables[s, i] = b
            pool[b, 0, :, :k[i * bs:(i + 1) * bs].shape[0]] = k[i * bs:(i + 1) * bs].transpose(1, 0, 2)
            pool[b, 1, :, :v[i * bs:(i + 1) * bs].shape[0]] = v[i * bs:(i + 1) * bs].transpose(1, 0, 2)
    return pool, tables


def prefill_is_masked_sdpa(prefill, seed=11):
    """Each sequence's chunk equals SDPA on its contiguous K/V with a causal
    mask aligned to the end of the context (is_causal when n = T)."""
    rng = np.random.default_rng(seed)
    lens, chunks, hq, hkv, d, bs = (40, 17, 64, 9), (40, 5, 20, 1), 8, 2, 16, 8
    ks = [rng.standard_normal((n, hkv, d)) for n in lens]
    vs = [rng.standard_normal((n, hkv, d)) for n in lens]
    pool, tables = _scatter(ks, vs, bs, seed)
    qstart = np.concatenate([[0], np.cumsum(chunks)])
    q = rng.standard_normal((int(qstart[-1]), hq, d))
    out = prefill(q, pool, tables, np.array(lens), qstart, 0.3)
    for s, (n, T) in enumerate(zip(lens, chunks)):
        kt = torch.from_numpy(ks[s]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        vt = torch.from_numpy(vs[s]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        qt = torch.from_numpy(q[qstart[s]:qstart[s + 1]]).permute(1, 0, 2)      # [Hq, T, D]
        if n == T:
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                                   scale=0.3)
        else:
            allowed = torch.arange(n)[None, :] <= (n - T + torch.arange(T))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed,
                                                                   scale=0.3)
        if not np.allclose(out[qstart[s]:qstart[s + 1]], ref.permute(1, 0, 2).numpy(),
                           rtol=0, atol=1e-12):
            return False
    return True


def prefill_single_token_is_decode(prefill, decode):
    """T = 1 for every sequence is the decode case, exactly."""
    rng = np.random.default_rng(12)
    kv = rng.standard_normal((12, 2, 2, 8, 16))
    bt = np.array([[3, 1, 7], [4, 0, 11]])
    lens = np.array([20, 9])
    q = rng.standard_normal((2, 4, 16))
    return bool(np.array_equal(prefill(q, kv, bt, lens, np.array([0, 1, 2]), 0.5),
                               decode(q, kv, bt, lens, 0.5)))


def chunked_equals_whole(prefill, seed=13):
    """Prefilling a prompt in two chunks (the second with the first as its
    past) gives the rows of prefilling it at once."""
    rng = np.random.default_rng(seed)
    n, t1, hq, hkv, d, bs = 37, 15, 4, 4, 8, 4
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    pool, tables = _scatter([k], [v], bs, seed)
    q = rng.standard_normal((n, hq, d))
    whole = prefill(q, pool, tables, np.array([n]), np.array([0, n]), 0.2)
    a = prefill(q[:t1], pool, tables, np.array([t1]), np.array([0, t1]), 0.2)
    b = prefill(q[t1:], pool, tables, np.array([n]), np.array([0, n - t1]), 0.2)
    return bool(np.allclose(np.concatenate([a, b]), whole, rtol=0, atol=1e-12))


def prefill_window_is_banded_sdpa(prefill, window, seed=14):
    """Under a window of W tokens each chunk equals SDPA on its contiguous
    K/V with a band mask: key t is allowed for the query at position p when
    p - W < t <= p (the causal mask cut to the last W tokens)."""
    rng = np.random.default_rng(seed)
    lens, chunks, hq, hkv, d, bs = (40, 17, 64, 9), (40, 5, 20, 1), 8, 2, 16, 8
    ks = [rng.standard_normal((n, hkv, d)) for n in lens]
    vs = [rng.standard_normal((n, hkv, d)) for n in lens]
    pool, tables = _scatter(ks, vs, bs, seed)
    qstart = np.concatenate([[0], np.cumsum(chunks)])
    q = rng.standard_normal((int(qstart[-1]), hq, d))
    out = prefill(q, pool, tables, np.array(lens), qstart, 0.3, window=window)
    for s, (n, T) in enumerate(zip(lens, chunks)):
        kt = torch.from_numpy(ks[s]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        vt = torch.from_numpy(vs[s]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        qt = torch.from_numpy(q[qstart[s]:qstart[s + 1]]).permute(1, 0, 2)      # [Hq, T, D]
        pos = (n - T + torch.arange(T))[:, None]
        t = torch.arange(n)[None, :]
        allowed = (t <= pos) & (t > pos - window)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed,
                                                               scale=0.3)
        if not np.allclose(out[qstart[s]:qstart[s + 1]], ref.permute(1, 0, 2).numpy(),
                           rtol=0, atol=1e-12):
            return False
    return True


def prefill_window_one_is_own_value_row(prefill):
    """W = 1: every query sees only its own token, so its output is that
    token's V row, exactly."""
    rng = np.random.default_rng(15)
    kv = rng.standard_normal((6, 2, 1, 4, 8))
    bt = np.array([[5, 2, 0]])
    q = rng.standard_normal((4, 2, 8))
    out = prefill(q, kv, bt, np.array([10]), np.array([0, 4]), 0.7, window=1)
    for i in range(4):
        p = 10 - 4 + i
        row = kv[bt[0, p // 4], 1, 0, p % 4]
        if not (np.array_equal(out[i, 0], row) and np.array_equal(out[i, 1], row)):
            return False
    return True


def i8_prefill_is_masked_sdpa_on_dequantised(prefill_i8, window=0, seed=18):
    """Chunked prefill over the INT8 pool equals SDPA over the dequantised
    contiguous K/V of each sequence with the end-aligned causal mask (cut to
    the last W tokens under a window), the codes and scales read through a
    random table: codes [block, K|V, head, row], scales [block, head, K|V,
    row]."""
    rng = np.random.default_rng(seed)
    lens, chunks, hq, hkv, d, bs = (40, 17, 64, 9), (40, 5, 20, 1), 8, 2, 16, 8
    nbs = [-(-n // bs) for n in lens]
    nb = sum(nbs) + 2
    codes = rng.integers(-127, 128, (nb, 2, hkv, bs, d)).astype(np.int8)
    scales = rng.uniform(0.001, 0.05, (nb, hkv, 2, bs)).astype(np.float32)
    perm = rng.permutation(nb)
    tables = np.full((len(lens), max(nbs)), -1)
    pos = 0
    for s, k in enumerate(nbs):
        tables[s, :k] = perm[pos:pos + k]
        pos += k
    qstart = np.concatenate([[0], np.cumsum(chunks)])
    q = rng.standard_normal((int(qstart[-1]), hq, d))
    out = prefill_i8(q, codes, scales, tables, np.array(lens), qstart, 0.3, window=window)
    for s, (n, T) in enumerate(zip(lens, chunks)):
        t = np.arange(n)
        blk = tables[s][t // bs]
        kk = codes[blk, 0, :, t % bs, :].astype(np.float64) * scales[blk, :, 0, t % bs][..., None]
        vv = codes[blk, 1, :, t % bs, :].astype(np.float64) * scales[blk, :, 1, t % bs][..., None]
        kt = torch.from_numpy(kk).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        vt = torch.from_numpy(vv).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        qt = torch.from_numpy(q[qstart[s]:qstart[s + 1]]).permute(1, 0, 2)
        p = (n - T + torch.arange(T))[:, None]
        allowed = torch.arange(n)[None, :] <= p
        if window > 0:
            allowed &= torch.arange(n)[None, :] > p - window
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed,
                                                               scale=0.3)
        if not np.allclose(out[qstart[s]:qstart[s + 1]], ref.permute(1, 0, 2).numpy(),
                           rtol=0, atol=1e-12):
            return False
    return True


def admission_threshold_keeps_one_shot_prompts_out(cls):
    """[KV2P] §4.3: with a minimum of two registrations before a block enters
    the cache, a prompt seen once stays private, a prompt seen twice is
    cached and hit by the third request, and a flood of one-shot prompts
    cannot evict it; the same flood with the threshold at 1 does."""
    bs, nb = 4, 12
    hot = list(range(100, 108))                         # two full blocks
    shots = [[1000 + 8 * k + j for j in range(8)] for k in range(20)]
    results = []
    for admit in (2, 1):
        m = cls(nb, bs)
        m.enable_prefix_cache(0, admit)
        seq = 0
        for _ in range(2):                               # the hot prompt, twice
            m.allocate_prompt(seq, hot)
            m.register(seq)
            m.free(seq)
            seq += 1
            if admit == 2 and _ == 0 and m.prefix_stats()[0] != 0:
                return False                             # cached after one sighting
        cached_after_two = m.prefix_stats()[0]
        for toks in shots:                               # one-shot flood
            m.allocate_prompt(seq, toks)
            m.register(seq)
            m.free(seq)
            seq += 1
        _, cached = m.allocate_prompt(seq, hot)
        results.append((cached_after_two, cached, m.prefix_stats()[6]))
    (c2, hit2, held2), (c1, hit1, held1) = results
    return c2 == 2 and hit2 == 8 and held2 == 2 + 2 * len(shots) and hit1 == 0 and held1 == 0


def admission_table_is_bounded(cls):
    """Keys below the threshold are remembered for at most num_blocks keys,
    the least recently seen dropped first: a key seen once, then pushed out
    by num_blocks other keys, starts counting again."""
    bs, nb = 2, 6

    def seen(m, seq, toks):
        m.allocate_prompt(seq, toks)
        m.register(seq)
        m.free(seq)

    m = cls(nb, bs)
    m.enable_prefix_cache(0, 2)
    seen(m, 0, [7, 7])
    for k in range(nb - 1):                              # room for the first key
        seen(m, 1 + k, [50 + k, 50 + k])
    seen(m, 10, [7, 7])                                  # second sighting: cached
    kept = m.prefix_stats()[0] == 1
    m = cls(nb, bs)
    m.enable_prefix_cache(0, 2)
    seen(m, 0, [7, 7])
    for k in range(nb):                                  # one more: the first is dropped
        seen(m, 1 + k, [50 + k, 50 + k])
    seen(m, 10, [7, 7])
    return kept and m.prefix_stats()[0] == 0
