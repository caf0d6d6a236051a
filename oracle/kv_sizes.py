"""Closed forms for KV-cache sizes (test infrastructure only).

The per-request KV size is 2 * L * H_kv * d_h * S * b bytes: L layers, H_kv
key/value heads, head dimension d_h, S tokens, b bytes per element, and the 2
for keys and values. The formula itself did not survive the pages' extraction;
its defining clause (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention &
Internals", section "Why the KV cache is the bottleneck") and the code that
evaluates it (same page, "How many blocks exist?"; modernaiengineering.com
lesson 13.15, listing "paged_kv.py") fix it. Values are pinned in
``tests/test_oracle_kv_sizes.py`` against figures printed on the pages.
"""
from __future__ import annotations


def kv_bytes(num_layers: int, num_kv_heads: int, head_size: int, num_tokens: int,
             elem_bytes: int) -> int:
    """Bytes of K and V for ``num_tokens`` tokens across ``num_layers`` layers."""
    return 2 * num_layers * num_kv_heads * head_size * num_tokens * elem_bytes


def bytes_per_block(block_size: int, num_layers: int, num_kv_heads: int, head_size: int,
                    elem_bytes: int) -> int:
    """Bytes of one KV block (``block_size`` token slots) across all layers."""
    return kv_bytes(num_layers, num_kv_heads, head_size, block_size, elem_bytes)


def blocks_in_pool(pool_bytes: int, block_bytes: int) -> int:
    """Whole blocks that fit in a pool of ``pool_bytes``."""
    return pool_bytes // block_bytes


def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """Blocks one sequence of ``num_tokens`` occupies: ceil(num_tokens / block_size)."""
    return -(-num_tokens // block_size)
