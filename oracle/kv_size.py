"""Closed forms for KV-cache sizes and block counts.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

* Per layer and per token the cache holds one K row and one V row of the
  model's key/value width ``d`` (``h`` heads of ``d/h``): ``2 d`` values; over
  ``L`` layers and ``S`` tokens in a ``e``-byte type that is ``L * 2 * d * S * e``
  bytes ([KVPA] §1.2, the memory formula and its 70B example).  With grouped
  KV heads the width is ``num_kv_heads * head_dim`` ([NANO] §1.2, the 7B
  example with 8 KV heads of 128).
* A sequence of ``n`` tokens needs ``ceil(n / block_size)`` blocks
  ([KVPA] §4.2: 100 tokens at block size 16 take 7 blocks, the last one
  partly filled; §5.3: after ``t`` tokens the next one needs
  ``ceil((t + 1) / block_size)`` blocks).
"""

from __future__ import annotations


def kv_values_per_token_layer(num_kv_heads, head_dim):
    """K and V values one token adds to one layer: 2 * Hkv * D."""
    return 2 * num_kv_heads * head_dim


def kv_bytes(num_layers, kv_width, num_tokens, dtype_bytes):
    """L * 2 * d * S * e bytes, with d = Hkv * D the key/value width."""
    return num_layers * 2 * kv_width * num_tokens * dtype_bytes


def blocks_needed(num_tokens, block_size):
    """ceil(num_tokens / block_size)."""
    return -(-num_tokens // block_size)


def decode_kv_bytes(context_lens, num_kv_heads, head_dim, dtype_bytes):
    """K+V bytes one decode step must read for one layer: sum_s n_s * 2 Hkv D e."""
    return sum(kv_bytes(1, num_kv_heads * head_dim, int(n), dtype_bytes) for n in context_lens)
