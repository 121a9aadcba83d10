"""Plain CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

This package is the correctness reference for the HIP library in
``paged_kv_cache_153_amd``.  It is written from the four source pages on the
KV cache and PagedAttention, in float64 NumPy, as slowly and plainly as the
definitions allow.  It shares no code, constants or helpers with the HIP path,
and the HIP path never imports it.

Who may use it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product path must never route
through it.

Sources cited in the modules (page title, then the section on that page):

* [KVPA]  "KV Cache与PagedAttention深度解析：vLLM内存管理革命" (iopencloud.com)
* [KV2P]  "KV Cache从原理到实战：大模型推理内存管理演进与优化" (xnwp.cn)
* [NANO]  the zwxr.cn nano-vllm walkthrough (the extract carries no title;
          cited by its own section numbers)
* [INFRA] "大模型 (LLM) 推理加速核心技术解析：从 KV Cache 到 PagedAttention 实战"
          (jsqmd.com)

Modules:

* ``attention``      — decode attention over a paged cache (definition),
                       causal multi-token (chunked prefill) attention, the
                       split-context partials and their log-sum-exp merge.
* ``cache``          — the slot-mapped K/V scatter and block copy-on-write.
* ``block_manager``  — a dict/list model of the host block manager.
* ``kv_size``        — closed forms for KV-cache sizes and block counts.
* ``quant``          — INT8 KV cache with one scale per 128-element group:
                       quantise on write, decode and prefill over the
                       dequantised pool.

Every function in these modules is pinned by a ``-m "not gpu"`` test against
something other than itself (closed forms, worked examples printed on the
pages, library routines on contiguous data, invariants).  No function is
"parity unpinned".
"""

from .attention import decode_ref, gather_sequence, split_ref, merge_ref, prefill_ref
from .cache import cache_write_ref
from .block_manager import BlockManagerModel, BlockManagerError
from .quant import (quantize_rows_ref, dequantize_ref, cache_write_i8_ref, decode_i8_ref,
                    prefill_i8_ref)
from . import kv_size

__all__ = [
    "decode_ref",
    "prefill_ref",
    "gather_sequence",
    "split_ref",
    "merge_ref",
    "cache_write_ref",
    "BlockManagerModel",
    "BlockManagerError",
    "kv_size",
    "quantize_rows_ref",
    "dequantize_ref",
    "cache_write_i8_ref",
    "decode_i8_ref",
    "prefill_i8_ref",
]
