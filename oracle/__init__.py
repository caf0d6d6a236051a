"""fp64 CPU oracle for paged decode attention and reshape_and_cache, and a
plain Python KV block pool with its step-input builder.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
path (``paged_kv_cache_150_amd``) and imports nothing from it.

What it computes is the plain definition the pages give: PagedAttention leaves
the arithmetic of attention unchanged and only indirects the addressing through
the block table (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention &
Internals", section "PagedAttention in one paragraph"). So the oracle gathers
each sequence's keys and values into contiguous arrays by logical position and
then evaluates softmax(q K^T * scale) V in float64.

Every function is pinned by ``tests/test_oracle_*.py`` against something
other than itself: brute-force contiguous attention, invariances, closed forms
and numbers printed on the pages (``tests/golden/``).
"""
from .paged_attention import (  # noqa: F401
    decode_values,
    gather_context,
    attention_contiguous,
    paged_decode,
    paged_decode_partitions,
    lse_merge,
    reshape_and_cache,
    copy_blocks,
)
from .kv_sizes import (  # noqa: F401
    kv_bytes,
    bytes_per_block,
    blocks_in_pool,
    blocks_for_tokens,
)
from .block_pool import (  # noqa: F401
    BlockPool,
    PoolError,
    prepare_step,
)
from .fp8 import (  # noqa: F401
    FP8_MAX,
    fp8_value,
    fp8_encode,
    quantize,
    dequantize,
    reshape_and_cache_fp8,
    paged_decode_fp8,
)
from .multi_query import paged_multi_query  # noqa: F401
