"""End-to-end parity of the decode step on the GPU against the oracle.

Both sides replay the same seeded operation sequence and the same new K/V
rows: sequences share a ref-counted prefix, one sequence is re-forked from a
random parent every step (so its first append copies the shared partial
block), every sequence appends one token, the rows are written, and decode
runs.  The HIP side uses the native block manager, pa_cache_write and
pa_decode; the oracle side uses its own block-manager model, cache write and
decode.  Checked every step: identical slots / copy pairs / tables,
bit-identical pools, decode within 5e-4."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_153_amd as pa
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_shared_prefix_fork_cow_steps(device, bs, kernel):
    print(f"pipeline bs={bs} kernel={kernel}", flush=True)
    S, Hq, Hkv, D, prefix, steps = 8, 8, 2, 128, 64, 12
    nb = 200
    gen = torch.Generator().manual_seed(bs)
    suffix = torch.randint(1, 70, (S - 1,), generator=gen).tolist()

    native, model = pa.BlockManager(nb, bs), oracle.BlockManagerModel(nb, bs)
    # pool contents: random everywhere, identical bits on both sides
    pool0 = synth.normal((nb, 2, Hkv, bs, D), torch.float16, synth._gen(3, "cpu"), "cpu")
    pool_ref = pool0.numpy().copy()
    pool_gpu = pool0.to(device)

    # prefix holder + S-1 sharers, then private suffixes token by token
    PREFIX = 1000
    native.allocate(PREFIX, prefix)
    model.allocate(PREFIX, prefix)
    pblocks = native.block_table(PREFIX)[0]
    assert pblocks == model.block_table(PREFIX)[0]
    for s in range(S - 1):
        native.share(s, pblocks, prefix)
        model.share(s, pblocks, prefix)
    remaining = list(suffix)
    while any(remaining):
        live = [s for s in range(S - 1) if remaining[s] > 0]
        slots_n, pairs_n = native.append_slots(live)
        want = [model.append_slot(s) for s in live]
        assert slots_n == [w[0] for w in want] and pairs_n == []
        for s in live:
            remaining[s] -= 1

    child = S - 1
    q = synth.normal((S, Hq, D), torch.float16, synth._gen(4, "cpu"), "cpu")
    total_cow = 0
    for step in range(steps):
        # re-fork the child from a parent that ends inside a block
        if child in model.tables:
            native.free(child)
            model.free(child)
        cands = [s for s in range(S - 1) if model.block_table(s)[1] % bs]
        parent = cands[int(torch.randint(0, len(cands), (1,), generator=gen))] if cands else 0
        native.fork(parent, child)
        model.fork(parent, child)
        order = [child] + list(range(S - 1))
        slots_n, pairs_n = native.append_slots(order)
        want = [model.append_slot(s) for s in order]
        assert slots_n == [w[0] for w in want]
        pairs_m = [(w[1], w[2]) for w in want if w[1] >= 0]
        assert pairs_n == pairs_m
        total_cow += len(pairs_n)

        k, v = synth.rows(S, Hkv, D, seed=100 + step)
        slots_m = np.array([w[0] for w in want], dtype=np.int64)
        pool_ref = oracle.cache_write_ref(pool_ref, k.numpy(), v.numpy(), slots_m,
                                          cow_pairs=pairs_m)
        d_pairs = (torch.tensor(pairs_n, dtype=torch.int32, device=device)
                   if pairs_n else None)
        pa.cache_write(k.to(device), v.to(device), pool_gpu,
                       torch.tensor(slots_n, dtype=torch.int64, device=device),
                       cow_pairs=d_pairs)

        mb = max(len(model.block_table(s)[0]) for s in order)
        rows, lens = native.block_tables(order, mb)
        bt_m = np.full((S, mb), -1, dtype=np.int64)
        cl_m = np.zeros(S, dtype=np.int64)
        for i, s in enumerate(order):
            t, n = model.block_table(s)
            bt_m[i, :len(t)] = t
            cl_m[i] = n
        assert np.array_equal(np.array(rows), bt_m) and list(cl_m) == lens
        bt = torch.tensor(rows, dtype=torch.int32)
        cl = torch.tensor(lens, dtype=torch.int32)
        out = pa.decode(q.to(device), pool_gpu, bt.to(device), cl.to(device),
                        max_context_len=int(cl.max()), kernel=kernel)
        torch.cuda.synchronize()
        got_pool = pool_gpu.cpu().numpy()
        assert np.array_equal(got_pool.view(np.uint16), pool_ref.view(np.uint16)), step
        want_out = oracle.decode_ref(q.numpy(), pool_ref, bt_m, cl_m, D ** -0.5)
        err = np.abs(out.cpu().numpy() - want_out).max()
        assert err <= 5e-4, (step, err)
    assert total_cow >= steps // 2   # the fork makes copy-on-write happen
    native.close()
