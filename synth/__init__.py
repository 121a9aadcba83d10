"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays them out; it holds none of the
attention, cache-write or block-manager arithmetic.  Both the oracle-side
tests and the HIP-side tests and bench take their inputs from here, so that
the two sides see the very same bits.

All values are i.i.d. normal, drawn as float32 with ``torch.randn`` from a
seeded ``torch.Generator`` on the requested device and rounded to the storage
dtype with round-to-nearest-even (``Tensor.to``).  Block tables hand out a
seeded random permutation of the physical pool in order, so each sequence's
blocks are scattered and non-contiguous; unused table entries are -1.

Named workloads (shapes of the LLaMA-2 7B / 70B layers the pages use as
examples; no weights are involved):

* ``tiny``          fp32, 4 seqs, 8 heads (MHA), head_dim 64, block 16,
                    context lengths 100, 37, 16, 1, a 64-block pool, scale 1/8.
* ``llama7b_mha``   fp16, 32 heads (MHA), head_dim 128, block 16, 32 seqs at
                    context 4096, a 9000-block pool.
* ``gqa7b``         fp16, 32 query / 8 KV heads, head_dim 128, block 16,
                    64 seqs with context lengths uniform on [128, 8192].
* ``llama70b``      fp16, 64 query / 8 KV heads, head_dim 128, block 16,
                    16 seqs at context 32768, values N(0, 0.5^2).
* ``shared_prefix`` fp16, 32 query / 8 KV heads, head_dim 128, block 8/16/32,
                    64 seqs sharing one 512-token prefix (the same physical
                    blocks in every table) plus private suffixes of uniform
                    1..2048 tokens.

Pools whose size the workload does not fix hold 1.1x the blocks the tables
use (rounded up), the same slack as 9000 blocks for 8192 used.

INT8 pools (``int8_pool``) keep a workload's queries, tables and lengths and
draw the pool itself as int8 codes plus one float32 scale per (block, K|V,
head, row): codes are rounded N(0, 42^2) draws clipped to [-127, 127] (about
the spread of rows whose largest value maps to 127), scales are uniform on
[0.01, 0.03] times the workload's standard deviation.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class DecodeInputs:
    name: str
    q: torch.Tensor              # [S, Hq, D]
    kv_cache: torch.Tensor       # [NB, 2, Hkv, bs, D]
    block_tables: torch.Tensor   # [S, MB] int32, -1 = unused
    context_lens: torch.Tensor   # [S] int32
    scale: float
    seed: int
    meta: dict = field(default_factory=dict)
    kv_scales: torch.Tensor = None   # INT8 pools: [NB, Hkv, 2, bs] float32

    @property
    def num_seqs(self):
        return self.q.shape[0]

    @property
    def num_q_heads(self):
        return self.q.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def num_kv_heads(self):
        return self.kv_cache.shape[2]

    @property
    def block_size(self):
        return self.kv_cache.shape[3]

    def to(self, device):
        return DecodeInputs(self.name, self.q.to(device), self.kv_cache.to(device),
                            self.block_tables.to(device), self.context_lens.to(device),
                            self.scale, self.seed, dict(self.meta),
                            None if self.kv_scales is None else self.kv_scales.to(device))


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, dtype, gen, device, std=1.0, chunk_rows=None):
    """N(0, std^2) float32 draws rounded to ``dtype``; drawn in chunks along dim 0
    when ``chunk_rows`` is given so that large pools need no float32 copy."""
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    step = rows if not chunk_rows else chunk_rows
    for lo in range(0, rows, step):
        hi = min(rows, lo + step)
        x = torch.randn((hi - lo,) + tuple(shape[1:]), generator=gen, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[lo:hi] = x.to(dtype)
    return out


def _tables_from_permutation(perm, blocks_per_seq, max_blocks):
    """Hand out ``perm`` in order: sequence s takes the next blocks_per_seq[s] ids."""
    tables = torch.full((len(blocks_per_seq), max(1, max_blocks)), -1, dtype=torch.int32)
    pos = 0
    for s, nb in enumerate(blocks_per_seq):
        tables[s, :nb] = perm[pos:pos + nb].to(torch.int32)
        pos += nb
    return tables


def make_decode_inputs(context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                       dtype="f16", seed=0, std=1.0, num_blocks=None, scale=None,
                       device="cpu", name="custom", max_blocks=None, fill_unused=None):
    """Random paged decode inputs.

    context_lens: list of ints.  ``num_blocks`` defaults to 1.1x the blocks used.
    ``fill_unused``: if set (e.g. float('nan')), every pool row that no
    sequence's context covers is overwritten with this value, so that a kernel
    that reads past a context shows it.
    """
    tdtype = DTYPES[dtype]
    lens = [int(n) for n in context_lens]
    per_seq = [-(-n // block_size) for n in lens]
    used = sum(per_seq)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(1.1 * used))
    if used > num_blocks:
        raise ValueError("pool too small for the context lengths")
    g_cpu = _gen(seed, "cpu")
    perm = torch.randperm(num_blocks, generator=g_cpu)
    mb = max(per_seq) if max_blocks is None else max_blocks
    tables = _tables_from_permutation(perm, per_seq, mb)
    g = _gen(seed + 1, device)
    q = normal((len(lens), num_q_heads, head_dim), tdtype, g, device, std)
    kv = normal((num_blocks, 2, num_kv_heads, block_size, head_dim), tdtype, g, device, std,
                chunk_rows=max(1, (1 << 26) // (2 * num_kv_heads * block_size * head_dim)))
    if fill_unused is not None:
        covered = torch.zeros((num_blocks, block_size), dtype=torch.bool)
        for s, n in enumerate(lens):
            for i in range(per_seq[s]):
                rows = min(block_size, n - i * block_size)
                covered[int(tables[s, i]), :rows] = True
        mask = (~covered).to(device)
        kv.permute(0, 3, 1, 2, 4)[mask] = torch.tensor(fill_unused, dtype=tdtype, device=device)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DecodeInputs(name, q, kv, tables.to(device),
                        torch.tensor(lens, dtype=torch.int32, device=device),
                        float(scale), seed,
                        {"num_blocks": num_blocks, "dtype": dtype, "std": std})


def int8_codes(shape, gen, device, code_std=42.0, chunk_rows=None):
    """Rounded N(0, code_std^2) draws clipped to [-127, 127], as int8."""
    out = torch.empty(shape, dtype=torch.int8, device=device)
    step = shape[0] if not chunk_rows else chunk_rows
    for lo in range(0, shape[0], step):
        hi = min(shape[0], lo + step)
        x = torch.randn((hi - lo,) + tuple(shape[1:]), generator=gen, device=device)
        out[lo:hi] = x.mul_(code_std).round_().clamp_(-127, 127).to(torch.int8)
    return out


def int8_pool(x, seed=None, fill_unused=None):
    """The same queries, tables and lengths as ``x`` over a freshly drawn INT8
    pool: codes [NB, 2, Hkv, bs, D] int8 and scales [NB, Hkv, 2, bs] float32.
    ``fill_unused`` (e.g. NaN) overwrites the scales of rows no context covers."""
    nb, two, hkv, bs, d = x.kv_cache.shape
    device = x.kv_cache.device
    seed = x.seed + 100 if seed is None else seed
    g = _gen(seed, device)
    codes = int8_codes((nb, two, hkv, bs, d), g, device,
                       chunk_rows=max(1, (1 << 26) // (2 * hkv * bs * d)))
    std = float(x.meta.get("std", 1.0))
    scales = (torch.rand((nb, hkv, two, bs), generator=g, device=device) * 0.02 + 0.01) * std
    if fill_unused is not None:
        covered = torch.zeros((nb, bs), dtype=torch.bool)
        tables = x.block_tables.cpu()
        for s, n in enumerate(x.context_lens.tolist()):
            for i in range(-(-n // bs)):
                covered[int(tables[s, i]), :min(bs, n - i * bs)] = True
        mask = (~covered).to(device)
        scales.permute(0, 3, 1, 2)[mask] = fill_unused
    q = x.q if x.q.dtype == torch.float16 else x.q.to(torch.float16)
    return DecodeInputs(x.name + "_i8", q, codes, x.block_tables, x.context_lens, x.scale,
                        x.seed, dict(x.meta, dtype="i8"), scales)


def tiny(seed=0, device="cpu", fill_unused=None):
    """4 seqs, MHA 8x64, fp32, block 16, lengths {100, 37, 16, 1}, 64-block pool.
    Tables: a seeded permutation of the 64 blocks, handed out in order."""
    return make_decode_inputs([100, 37, 16, 1], 8, 8, 64, 16, dtype="f32", seed=seed,
                              num_blocks=64, scale=1.0 / 8.0, device=device, name="tiny",
                              fill_unused=fill_unused)


def llama7b_mha(seed=0, device="cpu", num_seqs=32, context=4096):
    return make_decode_inputs([context] * num_seqs, 32, 32, 128, 16, dtype="f16", seed=seed,
                              num_blocks=9000 if (num_seqs, context) == (32, 4096) else None,
                              device=device, name="llama7b_mha")


def gqa_lengths(num_seqs, lo, hi, seed):
    g = _gen(seed + 7, "cpu")
    return torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist()


def gqa7b(seed=0, device="cpu", num_seqs=64, lo=128, hi=8192):
    return make_decode_inputs(gqa_lengths(num_seqs, lo, hi, seed), 32, 8, 128, 16,
                              dtype="f16", seed=seed, device=device, name="gqa7b")


def llama70b(seed=0, device="cpu", num_seqs=16, context=32768):
    return make_decode_inputs([context] * num_seqs, 64, 8, 128, 16, dtype="f16", seed=seed,
                              std=0.5, device=device, name="llama70b")


def shared_prefix(seed=0, device="cpu", block_size=16, num_seqs=64, prefix=512,
                  suffix_hi=2048, num_q_heads=32, num_kv_heads=8, head_dim=128,
                  spare_blocks=None):
    """64 sequences whose tables start with the same physical prefix blocks.

    The prefix blocks come first in the permutation, then each sequence's
    private suffix blocks.  ``spare_blocks`` extra free blocks are kept in the
    pool (default: 1.1x slack) for appends and copy-on-write.
    """
    g_cpu = _gen(seed + 11, "cpu")
    suffix = torch.randint(1, suffix_hi + 1, (num_seqs,), generator=g_cpu).tolist()
    pre_blocks = -(-prefix // block_size)
    suf_blocks = [-(-(prefix + n) // block_size) - pre_blocks for n in suffix]
    used = pre_blocks + sum(suf_blocks)
    num_blocks = math.ceil(1.1 * used) if spare_blocks is None else used + spare_blocks
    perm = torch.randperm(num_blocks, generator=_gen(seed, "cpu"))
    mb = pre_blocks + max(suf_blocks)
    tables = torch.full((num_seqs, mb), -1, dtype=torch.int32)
    pos = pre_blocks
    for s in range(num_seqs):
        tables[s, :pre_blocks] = perm[:pre_blocks].to(torch.int32)
        tables[s, pre_blocks:pre_blocks + suf_blocks[s]] = perm[pos:pos + suf_blocks[s]].to(torch.int32)
        pos += suf_blocks[s]
    g = _gen(seed + 1, device)
    tdtype = torch.float16
    q = normal((num_seqs, num_q_heads, head_dim), tdtype, g, device)
    kv = normal((num_blocks, 2, num_kv_heads, block_size, head_dim), tdtype, g, device,
                chunk_rows=max(1, (1 << 26) // (2 * num_kv_heads * block_size * head_dim)))
    lens = [prefix + n for n in suffix]
    return DecodeInputs(f"shared_prefix_bs{block_size}", q, kv, tables.to(device),
                        torch.tensor(lens, dtype=torch.int32, device=device),
                        1.0 / math.sqrt(head_dim), seed,
                        {"num_blocks": num_blocks, "dtype": "f16", "prefix_blocks": pre_blocks,
                         "free_blocks": [int(b) for b in perm[pos:].tolist()]})


def rows(num_tokens, num_kv_heads, head_dim, dtype="f16", seed=0, device="cpu", std=1.0):
    """New K and V rows for a cache write, each [T, Hkv, D]."""
    g = _gen(seed + 3, device)
    tdtype = DTYPES[dtype]
    k = normal((num_tokens, num_kv_heads, head_dim), tdtype, g, device, std)
    v = normal((num_tokens, num_kv_heads, head_dim), tdtype, g, device, std)
    return k, v


def distinct_slots(num_tokens, num_blocks, block_size, seed=0, skip_every=0):
    """``num_tokens`` distinct random slots in a pool of ``num_blocks`` blocks
    (int64); with ``skip_every = k > 0`` every k-th entry is -1."""
    g = _gen(seed + 5, "cpu")
    slots = torch.randperm(num_blocks * block_size, generator=g)[:num_tokens].to(torch.int64)
    if skip_every:
        slots[::skip_every] = -1
    return slots


WORKLOADS = {
    "tiny": tiny,
    "llama7b_mha": llama7b_mha,
    "gqa7b": gqa7b,
    "llama70b": llama70b,
    "shared_prefix": shared_prefix,
}
