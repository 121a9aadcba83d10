"""GPU parity for sliding-window decode ([KV2P] §7.2: each new token attends to
the last W tokens only) against the fp64 oracle, max-abs error <= 5e-4.

Every pool row that is not a key — past the context, or before the window —
holds NaN, so a kernel that reads or weighs a row outside [n - W, n) fails."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_153_amd as pa
import synth
from tests.full_oracle import assert_every_row

pytestmark = pytest.mark.gpu

TOL = 5e-4


def poison_before_window(x, window):
    """NaN in every row of sequence s that holds a token t < n - W (the
    sequences' blocks are disjoint in these inputs)."""
    bs = x.block_size
    kv = x.kv_cache
    for s, n in enumerate(x.context_lens.tolist()):
        lo = max(0, n - window)
        for t0 in range(0, lo, bs):
            b = int(x.block_tables[s, t0 // bs])
            rows = min(bs, lo - t0)
            kv[b, :, :, :rows] = float("nan")
    return x


def ref(x, window):
    return oracle.decode_ref(x.q.numpy(), x.kv_cache.numpy(), x.block_tables.numpy(),
                             x.context_lens.numpy(), x.scale, window=window)


def run(x, device, window, **kw):
    g = x.to(device)
    out = pa.decode(g.q, g.kv_cache, g.block_tables, g.context_lens, scale=x.scale,
                    max_context_len=int(x.context_lens.max()), sliding_window=window, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def kernels_for(x):
    ks = ["valu"]
    if x.kv_cache.dtype == torch.float16 and x.num_q_heads // x.num_kv_heads >= 2:
        ks.append("mfma")
    return ks


def check(x, device, window, parts=(-1, -2, 0, 16, 64, 512)):
    want = ref(x, window)
    assert np.isfinite(want).all()
    for kern in kernels_for(x):
        for part in parts:
            if part > 0 and (part % x.block_size or part % 16):
                continue
            print(f"  {x.name} W={window} kernel={kern} part={part}", flush=True)
            got = run(x, device, window, partition_size=part, kernel=kern)
            assert np.isfinite(got).all(), (kern, part)
            err = np.abs(got - want).max()
            assert err <= TOL, (kern, part, err)


LENS = [0, 1, 15, 16, 17, 31, 33, 100, 255, 256, 257, 700, 1500]


@pytest.mark.parametrize("window", [1, 7, 16, 17, 100, 256, 1000, 4096])
@pytest.mark.parametrize("bs", [8, 16, 32])
def test_window_ragged_gqa_f16(device, window, bs):
    x = synth.make_decode_inputs(LENS, 16, 4, 128, bs, dtype="f16", seed=31 + bs,
                                 fill_unused=float("nan"), name=f"gqa-bs{bs}")
    check(poison_before_window(x, window), device, window)


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 8, 8, 64), ("f16", 8, 8, 128),
                                            ("f16", 8, 4, 64), ("f32", 16, 2, 128)])
def test_window_shapes(device, dtype, hq, hkv, d):
    for window in (3, 32, 130):
        x = synth.make_decode_inputs([5, 48, 129, 600], hq, hkv, d, 16, dtype=dtype, seed=41,
                                     fill_unused=float("nan"), name=f"{dtype}-{hq}-{hkv}-{d}")
        check(poison_before_window(x, window), device, window, parts=(-1, -2, 64))


def test_window_one_returns_newest_value_row(device):
    """W = 1: a single key of weight one; the output is its V row (fp16 rows
    are exact in fp32)."""
    x = synth.make_decode_inputs([1, 9, 40, 333], 16, 4, 128, 16, dtype="f16", seed=43)
    lens = x.context_lens.tolist()
    for kern in kernels_for(x):
        for part in (-1, -2, 16):
            got = run(x, device, 1, partition_size=part, kernel=kern)
            for s, n in enumerate(lens):
                t = n - 1
                b = int(x.block_tables[s, t // 16])
                for h in range(16):
                    row = x.kv_cache[b, 1, h // 4, t % 16].double().numpy()
                    assert np.array_equal(got[s, h], row), (kern, part, s, h)


def test_window_at_least_context_equals_full_attention(device):
    """A window no shorter than every context changes nothing: bitwise equal
    to the call without a window for the same schedule."""
    x = synth.make_decode_inputs([37, 160, 511, 512], 32, 8, 128, 16, dtype="f16", seed=44)
    for kern in kernels_for(x):
        for part in (-1, -2, 64):
            a = run(x, device, 0, partition_size=part, kernel=kern)
            b = run(x, device, 512, partition_size=part, kernel=kern)
            c = run(x, device, 100000, partition_size=part, kernel=kern)
            assert np.array_equal(a, b) and np.array_equal(a, c), (kern, part)


@pytest.mark.parametrize("window", [4096, 1000])
def test_window_full_size_llama70b_every_row(device, window):
    """64 query / 8 KV heads, 16 x 32768 tokens, default launch; every
    (sequence, head) against the oracle over the window's blocks."""
    print(f"full-size llama70b W={window}", flush=True)
    x = synth.llama70b(seed=0, device=device)
    out = pa.decode(x.q, x.kv_cache, x.block_tables, x.context_lens, scale=x.scale,
                    max_context_len=int(x.context_lens.max()), sliding_window=window)
    torch.cuda.synchronize()
    assert_every_row(x, out, TOL, window=window)
    del x, out
    torch.cuda.empty_cache()
