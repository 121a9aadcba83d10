"""Checked mode (PA_CHECK=1): the device index arrays are copied to the host
and validated before anything is enqueued, so a bad block id, slot, copy
pair, length or chunk boundary is an error (PA_ERR_INVALID_ARG), not an
out-of-range read.  Every call below is refused on the host; the valid
calls beside them show the check lets good input through."""

import numpy as np
import pytest
import torch

import paged_kv_cache_153_amd as pa
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture
def checked(monkeypatch):
    monkeypatch.setenv("PA_CHECK", "1")


def _inputs(device):
    x = synth.make_decode_inputs([20, 5, 33], 8, 2, 64, 16, seed=1)
    return x, x.to(device)


def _refused(fn):
    with pytest.raises(pa.PAError) as e:
        fn()
    assert e.value.status == -1, e.value


def test_decode_checks_tables_and_lengths(device, checked):
    x, g = _inputs(device)
    ok = pa.decode(g.q, g.kv_cache, g.block_tables, g.context_lens, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(ok).all()
    bad = g.block_tables.clone()
    bad[2, 1] = x.kv_cache.shape[0] + 5                   # past the pool
    _refused(lambda: pa.decode(g.q, g.kv_cache, bad, g.context_lens, scale=x.scale))
    bad = g.block_tables.clone()
    bad[0, 0] = -1                                        # a hole inside the context
    _refused(lambda: pa.decode(g.q, g.kv_cache, bad, g.context_lens, scale=x.scale))
    lens = g.context_lens.clone()
    lens[1] = 40                                          # longer than max_context_len
    _refused(lambda: pa.decode(g.q, g.kv_cache, g.block_tables, lens, scale=x.scale,
                               max_context_len=33))


def test_cache_write_checks_slots_and_pairs(device, checked):
    x, g = _inputs(device)
    k, v = synth.rows(3, 2, 64, dtype="f16", seed=2)
    k, v = k.to(device), v.to(device)
    nslot = x.kv_cache.shape[0] * 16
    pa.cache_write(k, v, g.kv_cache, torch.tensor([0, 17, -1], device=device))
    torch.cuda.synchronize()
    _refused(lambda: pa.cache_write(k, v, g.kv_cache, torch.tensor([3, 3, 4], device=device)))
    _refused(lambda: pa.cache_write(k, v, g.kv_cache, torch.tensor([0, nslot, 1], device=device)))
    pairs = torch.tensor([[1, 2], [3, 2]], dtype=torch.int32, device=device)   # one dst twice
    _refused(lambda: pa.cache_write(k, v, g.kv_cache, torch.tensor([0, 1, 2], device=device),
                                    cow_pairs=pairs))
    pairs = torch.tensor([[1, 2], [2, 3]], dtype=torch.int32, device=device)   # dst is a src
    _refused(lambda: pa.cache_write(k, v, g.kv_cache, torch.tensor([0, 1, 2], device=device),
                                    cow_pairs=pairs))


def test_prefill_checks_chunks(device, checked):
    x, g = _inputs(device)
    q = synth.normal((12, 8, 64), torch.float16, synth._gen(3, "cpu"), "cpu").to(device)
    qs = torch.tensor([0, 4, 9, 12], dtype=torch.int32, device=device)
    out = pa.prefill(q, g.kv_cache, g.block_tables, g.context_lens, qs, scale=x.scale,
                     max_query_len=5)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    _refused(lambda: pa.prefill(q, g.kv_cache, g.block_tables, g.context_lens, qs,
                                scale=x.scale, max_query_len=4))        # a chunk of 5 > 4
    bad_qs = torch.tensor([1, 4, 9, 12], dtype=torch.int32, device=device)
    _refused(lambda: pa.prefill(q, g.kv_cache, g.block_tables, g.context_lens, bad_qs,
                                scale=x.scale, max_query_len=5))
    bad = g.block_tables.clone()
    bad[1, 0] = 10 ** 6
    _refused(lambda: pa.prefill(q, g.kv_cache, bad, g.context_lens, qs, scale=x.scale,
                                max_query_len=5))
