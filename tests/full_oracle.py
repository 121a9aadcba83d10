"""The fp64 oracle over every (sequence, head) of a full-size workload.

Each sequence's blocks (only those holding its keys: the window's under a
sliding window) are copied to host memory on their own and renumbered, and
the oracle runs on them in a pool of worker threads with BLAS limited to one
thread each (NumPy releases the GIL inside its array operations).  A full
7B or 70B layer takes a few seconds this way, so full-size parity tests can
compare every output row instead of a sample.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _host_sequence(x, s, window):
    """(q [1, Hq, D], blocks, scales or None, table [1, nblk], n') on the host
    for sequence s: the blocks from the first one holding a key onwards."""
    bs = x.block_size
    n = int(x.context_lens[s])
    lo_blk = max(0, n - window) // bs if window > 0 else 0
    nblk = -(-n // bs) - lo_blk
    ids = x.block_tables[s, lo_blk:lo_blk + nblk].long()
    blocks = x.kv_cache[ids].cpu().numpy()
    scales = None if x.kv_scales is None else x.kv_scales[ids].cpu().numpy()
    return (x.q[s:s + 1].cpu().numpy(), blocks, scales, np.arange(nblk)[None],
            n - lo_blk * bs)


def every_row(x, window=0):
    """Oracle output [S, Hq, D] float64 for the decode inputs ``x`` (device
    tensors; an INT8 pool when ``x.kv_scales`` is set)."""
    from threadpoolctl import threadpool_limits

    def one(item):
        q, blocks, scales, table, n = item
        if scales is None:
            return oracle.decode_ref(q, blocks, table, np.array([n]), x.scale, window=window)
        return oracle.decode_i8_ref(q, blocks, scales, table, np.array([n]), x.scale,
                                    window=window)

    S, Hq, D = x.num_seqs, x.num_q_heads, x.head_dim
    out = np.zeros((S, Hq, D))
    workers = _workers()
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        pending = []
        for s in range(S):
            pending.append((s, ex.submit(one, _host_sequence(x, s, window))))
            while len(pending) >= 2 * workers:      # bound the host copies in flight
                s0, f = pending.pop(0)
                out[s0] = f.result()[0]
        for s0, f in pending:
            out[s0] = f.result()[0]
    return out


def assert_every_row(x, out, tol, window=0):
    """Every output row of ``out`` (device, [S, Hq, D]) within ``tol`` (max
    abs) of the oracle; names the worst (sequence, head) on failure."""
    want = every_row(x, window)
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - want).max(axis=2)
    s, h = np.unravel_index(int(np.argmax(err)), err.shape)
    assert err[s, h] <= tol, (int(s), int(h), float(err[s, h]))
    return float(err.max())


def every_prefill_row(x, q, qstart, window=0, rows=16):
    """Oracle output [total_q, Hq, D] float64 of a chunked prefill (``x`` and
    ``q`` on the device; an INT8 pool when ``x.kv_scales`` is set): each
    sequence's blocks are copied to host memory once, and its chunk is cut
    into groups of ``rows`` query rows, each the last rows of a context that
    ends at its last row, computed in a pool of worker threads."""
    from threadpoolctl import threadpool_limits

    bs = x.block_size
    lens = x.context_lens.tolist()
    host = []
    for s, n in enumerate(lens):
        nblk = -(-n // bs)
        ids = x.block_tables[s, :nblk].long()
        host.append((x.kv_cache[ids].cpu().numpy(),
                     None if x.kv_scales is None else x.kv_scales[ids].cpu().numpy()))
    qh = q.cpu().numpy()
    jobs = []
    for s, n in enumerate(lens):
        q0, q1 = int(qstart[s]), int(qstart[s + 1])
        T = q1 - q0
        for i0 in range(0, T, rows):
            jobs.append((s, n, T, q0, i0, min(T, i0 + rows)))

    def one(job):
        s, n, T, q0, i0, i1 = job
        blocks, scales = host[s]
        args = (np.arange(blocks.shape[0])[None], np.array([n - T + i1]),
                np.array([0, i1 - i0]), x.scale)
        if scales is None:
            return oracle.prefill_ref(qh[q0 + i0:q0 + i1], blocks, *args, window=window)
        return oracle.prefill_i8_ref(qh[q0 + i0:q0 + i1], blocks, scales, *args, window=window)

    out = np.zeros(qh.shape)
    with threadpool_limits(1), ThreadPoolExecutor(_workers()) as ex:
        for job, res in zip(jobs, ex.map(one, jobs)):
            s, n, T, q0, i0, i1 = job
            out[q0 + i0:q0 + i1] = res
    return out


def assert_every_prefill_row(x, q, qstart, out, tol, window=0):
    """Every row of ``out`` (device, [total_q, Hq, D]) within ``tol`` of the
    oracle; names the worst (row, head) on failure."""
    want = every_prefill_row(x, q, qstart, window)
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - want).max(axis=2)
    r, h = np.unravel_index(int(np.argmax(err)), err.shape)
    assert err[r, h] <= tol, (int(r), int(h), float(err[r, h]))
    return float(err.max())
