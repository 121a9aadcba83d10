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
from tests.full_oracle import assert_every_row

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
