"""GPU parity for the INT8 KV cache ([KV2P] §5.2: INT8 codes with one scale per
128-element group).

* pa_cache_write into an INT8 pool: codes and scales bit-exact against the
  oracle's quantiser (the decisions are float32 on both sides), including
  ties, zero rows, copy-on-write pairs and skipped slots.
* pa_decode over an INT8 pool: max-abs error <= 5e-4 against the fp64
  oracle's decode over the dequantised pool, for both kernel families, every
  schedule, every block size and head_dim, windows, and full-size workloads
  on every output row.  Scales of rows outside every context are NaN, so a
  kernel that weighs such a row fails.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_153_amd as pa
import synth
from tests.full_oracle import assert_every_prefill_row, assert_every_row

pytestmark = pytest.mark.gpu

TOL = 5e-4


def ref(x, window=0):
    return oracle.decode_i8_ref(x.q.numpy(), x.kv_cache.numpy(), x.kv_scales.numpy(),
                                x.block_tables.numpy(), x.context_lens.numpy(), x.scale,
                                window=window)


def run(x, device, **kw):
    g = x.to(device)
    out = pa.decode(g.q, g.kv_cache, g.block_tables, g.context_lens, scale=x.scale,
                    max_context_len=int(x.context_lens.max()), kv_scales=g.kv_scales, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def kernels_for(x):
    return ["valu", "mfma"] if x.num_q_heads // x.num_kv_heads >= 2 else ["valu"]


def check(x, device, parts=(-1, -2, 0, 16, 64), window=0, kernels=None):
    want = ref(x, window)
    assert np.isfinite(want).all()
    for kern in kernels or kernels_for(x):
        for part in parts:
            if part > 0 and (part % x.block_size or part % 16):
                continue
            print(f"  {x.name} kernel={kern} part={part} W={window}", flush=True)
            got = run(x, device, partition_size=part, kernel=kern, sliding_window=window)
            assert np.isfinite(got).all(), (kern, part)
            err = np.abs(got - want).max()
            assert err <= TOL, (kern, part, err)


# --------------------------------------------------------------------------
# cache write: quantisation on the way in, bit-exact
# --------------------------------------------------------------------------
def _write_case(device, T, hkv, d, bs, nb, seed, cow=(), skip_every=0, special=False):
    k, v = synth.rows(T, hkv, d, dtype="f16", seed=seed, std=2.0)
    if special:
        k[0] = 0                                                     # zero row
        k[1, :, :8] = torch.tensor([127, 2.5, -2.5, 3.5, 0.5, -0.5, 1.5, -1.5],
                                   dtype=torch.float16)              # ties at scale 1
        k[1, :, 8:] = 0
        v[2] = torch.tensor(60000.0, dtype=torch.float16)            # large, equal values
        v[3, :, 0] = -900.0                                          # outlier
    slots = synth.distinct_slots(T, nb, bs, seed=seed, skip_every=skip_every)
    base = synth.int8_pool(synth.make_decode_inputs([1], 2 * hkv, hkv, d, bs, num_blocks=nb,
                                                    seed=seed), seed=seed + 9)
    codes, scales = base.kv_cache, base.kv_scales
    want_c, want_s = oracle.cache_write_i8_ref(codes.numpy(), scales.numpy(), k.numpy(),
                                               v.numpy(), slots.numpy(), cow)
    c_dev, s_dev = codes.to(device), scales.to(device)
    pairs = torch.tensor(cow, dtype=torch.int32, device=device).reshape(-1, 2) if cow else None
    pa.cache_write(k.to(device), v.to(device), c_dev, slots.to(device), cow_pairs=pairs,
                   kv_scales=s_dev)
    torch.cuda.synchronize()
    assert np.array_equal(c_dev.cpu().numpy(), want_c)
    assert np.array_equal(s_dev.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [8, 16, 32])
def test_cache_write_quantises_bit_exact(device, d, bs):
    print(f"i8 write d={d} bs={bs}", flush=True)
    _write_case(device, 300, 4, d, bs, nb=64 if bs == 32 else 128, seed=d + bs, skip_every=7)


def test_cache_write_ties_zero_rows_and_outliers(device):
    _write_case(device, 16, 2, 128, 16, nb=8, seed=3, special=True)


def test_cache_write_copy_on_write_moves_scales(device):
    _write_case(device, 5, 2, 64, 16, nb=12, seed=4, cow=[(1, 2), (5, 7), (0, 9)])


def test_cache_write_many_tokens(device):
    _write_case(device, 5000, 8, 128, 16, nb=400, seed=5)


# --------------------------------------------------------------------------
# decode over an INT8 pool
# --------------------------------------------------------------------------
def _ragged(bs, d, hq, hkv, seed, lens=(0, 1, 15, 16, 17, 100, 255, 700, 1500)):
    x = synth.make_decode_inputs(list(lens), hq, hkv, d, bs, dtype="f16", seed=seed,
                                 name=f"i8-bs{bs}-d{d}-{hq}/{hkv}")
    return synth.int8_pool(x, fill_unused=float("nan"))


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (16, 4), (16, 2)])
def test_decode_ragged(device, bs, d, hq, hkv):
    check(_ragged(bs, d, hq, hkv, seed=bs + d + hq), device)


@pytest.mark.parametrize("window", [1, 17, 300])
def test_decode_with_window(device, window):
    x = _ragged(16, 128, 32, 8, seed=51)
    check(x, device, parts=(-1, -2, 0, 64), window=window)


def test_decode_single_token_is_its_value_row(device):
    """n = 1: one key of weight one; the output is its dequantised V row
    (to the float32 product of code and scale, and the 16-bit split of the
    weight in the matrix-core kernel)."""
    x = synth.int8_pool(synth.make_decode_inputs([1, 1, 1], 16, 4, 128, 16, seed=52))
    for kern in ("valu", "mfma"):
        for part in (-1, -2):
            got = run(x, device, partition_size=part, kernel=kern)
            for s in range(3):
                b = int(x.block_tables[s, 0])
                for h in range(16):
                    want = (x.kv_cache[b, 1, h // 4, 0].double() *
                            float(x.kv_scales[b, h // 4, 1, 0])).numpy()
                    assert np.abs(got[s, h] - want).max() <= 2e-5 * np.abs(want).max() + 1e-7


def test_decode_large_scales(device):
    """Scales up to ~500 (rows with values near the f16 maximum): the weights
    times V scales must not overflow inside the kernels."""
    x = _ragged(16, 128, 16, 2, seed=53, lens=(3, 90, 400))
    x.kv_scales[:, :, 1] *= 20000.0
    want = ref(x)
    for kern in ("valu", "mfma"):
        for part in (-1, -2, 64):
            got = run(x, device, partition_size=part, kernel=kern)
            assert np.isfinite(got).all()
            assert np.abs(got - want).max() <= TOL * np.abs(want).max(), (kern, part)


def test_pipeline_write_then_decode(device):
    """Write fresh f16 rows into an INT8 pool through pa_cache_write, then
    decode; the oracle takes the same rows through its own quantiser."""
    lens = [40, 129, 300]
    x = synth.int8_pool(synth.make_decode_inputs(lens, 32, 8, 128, 16, seed=54))
    # the last token of each sequence is rewritten from f16 rows
    k, v = synth.rows(len(lens), 8, 128, dtype="f16", seed=55)
    slots = torch.tensor([int(x.block_tables[s, (n - 1) // 16]) * 16 + (n - 1) % 16
                          for s, n in enumerate(lens)], dtype=torch.int64)
    c_ref, s_ref = oracle.cache_write_i8_ref(x.kv_cache.numpy(), x.kv_scales.numpy(), k.numpy(),
                                             v.numpy(), slots.numpy())
    want = oracle.decode_i8_ref(x.q.numpy(), c_ref, s_ref, x.block_tables.numpy(),
                                np.array(lens), x.scale)
    g = x.to(device)
    pa.cache_write(k.to(device), v.to(device), g.kv_cache, slots.to(device), kv_scales=g.kv_scales)
    for kern in ("valu", "mfma"):
        out = pa.decode(g.q, g.kv_cache, g.block_tables, g.context_lens, scale=x.scale,
                        kv_scales=g.kv_scales, kernel=kern)
        torch.cuda.synchronize()
        assert np.abs(out.cpu().numpy() - want).max() <= TOL, kern


@pytest.mark.parametrize("name", ["llama7b_mha", "gqa7b", "llama70b"])
def test_full_size_every_row(device, name):
    """Full workload shapes over INT8 pools, default launch; every
    (sequence, head) against the oracle over the dequantised pool."""
    print(f"full-size i8 {name}", flush=True)
    x = synth.int8_pool(synth.WORKLOADS[name](seed=0, device=device))
    out = pa.decode(x.q, x.kv_cache, x.block_tables, x.context_lens, scale=x.scale,
                    max_context_len=int(x.context_lens.max()), kv_scales=x.kv_scales)
    torch.cuda.synchronize()
    assert_every_row(x, out, TOL)
    del x, out
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# chunked prefill over an INT8 pool ([KV2P] §5.2 cache, §5.4 chunked prefill)
# --------------------------------------------------------------------------
def _i8_prefill_inputs(lens, chunks, hq, hkv, d, bs, seed, window=0, scale=None, code_std=1.0):
    """An INT8 pool whose scales are NaN outside every context and before
    every query's window, and f16 queries of the chunks."""
    base = synth.make_decode_inputs(lens, hq, hkv, d, bs, dtype="f16", seed=seed, scale=scale,
                                    std=code_std)
    x = synth.int8_pool(base, fill_unused=float("nan"))
    if window:
        for s, (n, T) in enumerate(zip(lens, chunks)):
            lo = max(0, n - T - window + 1) if T else n
            for t0 in range(0, lo, bs):
                b = int(x.block_tables[s, t0 // bs])
                x.kv_scales[b, :, :, :min(bs, lo - t0)] = float("nan")
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = synth.normal((int(qs[-1]), hq, d), torch.float16, synth._gen(seed + 50, "cpu"), "cpu",
                     code_std)
    return x, q, qs


def _i8_prefill(x, q, qs, device, window=0):
    g = x.to(device)
    out = pa.prefill(q.to(device), g.kv_cache, g.block_tables, g.context_lens,
                     torch.from_numpy(qs).to(device), scale=x.scale,
                     max_query_len=max(1, int(np.diff(qs).max())), sliding_window=window,
                     kv_scales=g.kv_scales)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _i8_prefill_ref(x, q, qs, window=0):
    return oracle.prefill_i8_ref(q.numpy(), x.kv_cache.numpy(), x.kv_scales.numpy(),
                                 x.block_tables.numpy(), x.context_lens.numpy(), qs, x.scale,
                                 window=window)


@pytest.mark.parametrize("window", [0, 7, 100])
@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 8), (64, 16, 2), (128, 16, 4), (128, 32, 4)])
def test_prefill_ragged_chunks(device, window, bs, d, hq, hkv):
    lens = [1, 17, 40, 100, 33, 300, 64, 500]
    chunks = [1, 17, 9, 100, 1, 37, 64, 129]
    x, q, qs = _i8_prefill_inputs(lens, chunks, hq, hkv, d, bs, seed=bs + d + hq + window,
                                  window=window)
    print(f"  i8 prefill W={window} bs={bs} d={d} {hq}/{hkv}", flush=True)
    want = _i8_prefill_ref(x, q, qs, window)
    assert np.isfinite(want).all()
    got = _i8_prefill(x, q, qs, device, window)
    assert np.isfinite(got).all()
    assert np.abs(got - want).max() <= TOL


def test_prefill_single_token_chunks_match_i8_decode(device):
    x, q, qs = _i8_prefill_inputs([50, 7, 129, 700], [1, 1, 1, 1], 32, 8, 128, 16, seed=91)
    got = _i8_prefill(x, q, qs, device)
    g = x.to(device)
    dec = pa.decode(q.to(device), g.kv_cache, g.block_tables, g.context_lens, scale=x.scale,
                    partition_size=-1, kv_scales=g.kv_scales)
    torch.cuda.synchronize()
    assert np.abs(got - dec.cpu().numpy()).max() <= 1e-5
    assert np.abs(got - _i8_prefill_ref(x, q, qs)).max() <= TOL


def test_prefill_peaked_scores_move_the_reference(device):
    """Scale 1 and wide values: later keys pass the first step's scores by
    far more than 2^8, so the kernel rescales live accumulators; every row
    against the oracle."""
    lens, chunks = [300, 97, 700], [300, 40, 129]
    x, q, qs = _i8_prefill_inputs(lens, chunks, 32, 4, 128, 16, seed=92, scale=1.0,
                                  code_std=3.0)
    k = oracle.dequantize_ref(x.kv_cache.numpy()[:, 0], x.kv_scales.numpy()[:, :, 0])
    jumps = 0
    for s, (n, T) in enumerate(zip(lens, chunks)):
        t = np.arange(n)
        blk = x.block_tables.numpy()[s][t // 16]
        ks = k[blk, :, t % 16, :]                       # [n, Hkv, D]
        for i in range(0, T, 7):
            p = n - T + i
            if p < 32:
                continue
            for h in range(0, 32, 5):
                z = ks[:p + 1, h // 8] @ q[qs[s] + i, h].double().numpy() / np.log(2)
                jumps += int(z[32:].max() > z[:32].max() + 8)
    assert jumps >= 20
    got = _i8_prefill(x, q, qs, device)
    assert np.isfinite(got).all()
    assert np.abs(got - _i8_prefill_ref(x, q, qs)).max() <= TOL


def test_prefill_after_cache_write_of_the_chunk(device):
    """The chunk's rows are quantised into the pool by pa_cache_write, then
    attended to by pa_prefill; the oracle takes the same f16 rows through its
    own quantiser and prefill."""
    lens, chunks, bs = [200, 64, 333], [50, 64, 1], 16
    x, q, qs = _i8_prefill_inputs(lens, chunks, 16, 4, 128, bs, seed=93)
    rows = int(qs[-1])
    k, v = synth.rows(rows, 4, 128, dtype="f16", seed=94)
    bt = x.block_tables.numpy()
    slots = []
    for s, (n, T) in enumerate(zip(lens, chunks)):
        for p in range(n - T, n):
            slots.append(int(bt[s, p // bs]) * bs + p % bs)
    slots = torch.tensor(slots, dtype=torch.int64)
    codes, scales = oracle.cache_write_i8_ref(x.kv_cache.numpy(), x.kv_scales.numpy(),
                                              k.numpy(), v.numpy(), slots.numpy())
    want = oracle.prefill_i8_ref(q.numpy(), codes, scales, bt, np.array(lens), qs, x.scale)
    g = x.to(device)
    pa.cache_write(k.to(device), v.to(device), g.kv_cache, slots.to(device),
                   kv_scales=g.kv_scales)
    out = pa.prefill(q.to(device), g.kv_cache, g.block_tables, g.context_lens,
                     torch.from_numpy(qs).to(device), scale=x.scale, max_query_len=64,
                     kv_scales=g.kv_scales)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().numpy().astype(np.float64) - want).max() <= TOL


@pytest.mark.parametrize("window", [0, 1024])
def test_prefill_long_chunk_70b_heads_every_row(device, window):
    """A 1536-token chunk at context 3000 and a fresh 700-token prompt, 64 q /
    8 KV heads over an INT8 pool: every row against the oracle."""
    lens, chunks = [3000, 700], [1536, 700]
    x, q, qs = _i8_prefill_inputs(lens, chunks, 64, 8, 128, 16, seed=95, window=window)
    g = x.to(device)
    out = pa.prefill(q.to(device), g.kv_cache, g.block_tables, g.context_lens,
                     torch.from_numpy(qs).to(device), scale=x.scale, max_query_len=1536,
                     sliding_window=window, kv_scales=g.kv_scales)
    torch.cuda.synchronize()
    assert_every_prefill_row(g, q, qs, out, TOL, window=window)


def test_prefill_gqa_chunk_every_row(device):
    """The benchmarked prefill (8 x 512-token chunks at context 4096, 32 q /
    8 KV heads) over an INT8 pool: every row against the oracle."""
    lens, chunks = [4096] * 8, [512] * 8
    x, q, qs = _i8_prefill_inputs(lens, chunks, 32, 8, 128, 16, seed=96)
    g = x.to(device)
    out = pa.prefill(q.to(device), g.kv_cache, g.block_tables, g.context_lens,
                     torch.from_numpy(qs).to(device), scale=x.scale, max_query_len=512,
                     kv_scales=g.kv_scales)
    torch.cuda.synchronize()
    assert_every_prefill_row(g, q, qs, out, TOL)
