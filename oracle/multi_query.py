"""Multi-query paged attention: several new query tokens per sequence (a
prompt chunk, or the k+1 positions a speculative step verifies), each attending
causally over the sequence's paged context (test infrastructure only).

The pages: one kernel serves any mix of prefill chunks and one-token decodes
(llm-stack-book 7.3 "vLLM: Architecture, PagedAttention & Internals", sections
"Prefill, decode, and chunked prefill" and "The forward step in detail"), and a
speculative step runs the target model on all k+1 positions at once (same
page, "Speculative decoding"). The new tokens' K/V are in the cache before
attention runs (the forward step scatters them first), so with n tokens
stored and q of them new, query token j sits at position n - q + j and sees
the keys at positions 0 .. n - q + j: everything before it and itself.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import attention_contiguous, decode_values, gather_context


def paged_multi_query(query, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                      scale: float, dtype: str, block_size: int = 16, kv_dtype: str | None = None):
    """query [T, H_q, d_h] holds the new tokens of every sequence, sequence i's
    at rows query_start_loc[i] .. query_start_loc[i+1]. Returns (out [T, H_q,
    d_h], lse [T, H_q]) in float64. A token whose position would be negative
    (more new tokens than stored ones) sees no key: out 0, lse -inf."""
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    T, Hq, d = query.shape
    out = np.zeros((T, Hq, d))
    lse = np.full((T, Hq), -np.inf)
    loc = np.asarray(query_start_loc, dtype=np.int64)
    for i in range(len(loc) - 1):
        n = int(context_lens[i])
        q0, q1 = int(loc[i]), int(loc[i + 1])
        Kc, Vc = gather_context(key_cache, value_cache, block_tables[i], n, block_size)
        Kf, Vf = decode_values(Kc, kv_dtype), decode_values(Vc, kv_dtype)
        for t in range(q0, q1):
            pos = n - (q1 - q0) + (t - q0)
            if pos < 0:
                continue
            out[t], lse[t] = attention_contiguous(decode_values(query[t], dtype), Kf[:pos + 1], Vf[:pos + 1],
                                                  scale)
    return out, lse
