"""fp64 reference for the paged decode hot path (test infrastructure only).

Definitions follow the pages:

* Block table and slot addressing: token position ``pos`` of a sequence lives
  in logical block ``pos // block_size`` at offset ``pos % block_size``; the
  block table maps the logical block to a physical block id, and the flat slot
  is ``physical * block_size + offset`` (llm-stack-book 7.3 "vLLM:
  Architecture, PagedAttention & Internals", section "The forward step in
  detail").
* Attention itself is unchanged by paging; only the addressing is indirected
  (same page, section "PagedAttention in one paragraph"). GQA: H_q query heads
  share H_kv key/value heads (same page, section "Why the KV cache is the
  bottleneck"); query head h reads kv head ``h // (H_q / H_kv)`` (reading:
  contiguous groups).
* The softmax normaliser can be carried as a running maximum and sum, which is
  what lets a kernel stream a sequence piecewise (stanleyjacob.dev "vLLM",
  Part IV "Stage 6: The forward pass" and Part V "The attention backend
  dispatch layer"); a context split into partitions is merged exactly with
  log-sum-exp weights.
* reshape_and_cache: the freshly computed K and V of each token are scattered
  into the cache at its slot (llm-stack-book 7.3, "The forward step in
  detail").
"""
from __future__ import annotations

import numpy as np


def decode_values(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.

    ``bf16`` arrays hold raw bfloat16 bits (uint16): widen to the upper half of
    an IEEE float32 word, then to float64. ``f32`` arrays are float32.
    """
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def gather_context(key_cache: np.ndarray, value_cache: np.ndarray, block_table_row: np.ndarray,
                   n: int, block_size: int):
    """Contiguous K and V ([n, H_kv, d_h], stored dtype) of one sequence.

    Position tau reads physical block ``block_table_row[tau // block_size]`` at
    offset ``tau % block_size``. Table entries past ``ceil(n / block_size)`` are
    never looked at.
    """
    tau = np.arange(n, dtype=np.int64)
    logical = tau // block_size
    offset = tau % block_size
    physical = np.asarray(block_table_row, dtype=np.int64)[logical]
    return key_cache[physical, offset], value_cache[physical, offset]


def attention_contiguous(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Textbook attention of one query position over a contiguous context.

    q: [H_q, d_h] float64; K, V: [n, H_kv, d_h] float64.
    Returns (out [H_q, d_h], lse [H_q]) with lse = ln sum_tau exp(s_tau).
    An empty context (n = 0) gives out = 0 and lse = -inf.
    """
    Hq, d = q.shape
    n, Hkv, _ = K.shape
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    g = Hq // Hkv
    out = np.zeros((Hq, d), dtype=np.float64)
    lse = np.full(Hq, -np.inf, dtype=np.float64)
    if n == 0:
        return out, lse
    # [H_kv, g, d] x [H_kv, d, n] -> scores [H_kv, g, n]
    qg = q.reshape(Hkv, g, d)
    s = scale * np.matmul(qg, K.transpose(1, 2, 0))
    m = s.max(axis=2, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=2, keepdims=True)
    o = np.matmul(w, V.transpose(1, 0, 2)) / l          # [H_kv, g, d]
    out[:] = o.reshape(Hq, d)
    lse[:] = (m + np.log(l)).reshape(Hq)
    return out, lse


def paged_decode(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                 dtype: str, block_size: int = 16, seqs=None, kv_dtype: str | None = None):
    """Decode-step attention for every sequence, reading K/V through the block table.

    Returns (out [S, H_q, d_h], lse [S, H_q]) in float64. ``seqs`` optionally
    restricts the work to a subset of sequence indices (the rest stay NaN).
    ``kv_dtype`` names the caches' storage when it differs from the query's
    ("f64": values already decoded, as for FP8 caches).
    """
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    S, Hq, d = query.shape
    out = np.full((S, Hq, d), np.nan, dtype=np.float64)
    lse = np.full((S, Hq), np.nan, dtype=np.float64)
    idx = range(S) if seqs is None else seqs
    for i in idx:
        n = int(context_lens[i])
        Kc, Vc = gather_context(key_cache, value_cache, block_tables[i], n, block_size)
        q = decode_values(query[i], dtype)
        out[i], lse[i] = attention_contiguous(q, decode_values(Kc, kv_dtype),
                                              decode_values(Vc, kv_dtype), scale)
    return out, lse


def paged_decode_partitions(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                            block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                            dtype: str, partition_size: int, num_parts: int,
                            block_size: int = 16, seqs=None):
    """Per-partition attention: partition p covers positions [p*P, min((p+1)*P, n)).

    Returns (o_parts [S, H_q, num_parts, d_h], lse_parts [S, H_q, num_parts]);
    each o_p is normalised within its partition, empty partitions have
    o_p = 0 and lse_p = -inf.
    """
    S, Hq, d = query.shape
    o_parts = np.zeros((S, Hq, num_parts, d), dtype=np.float64)
    lse_parts = np.full((S, Hq, num_parts), -np.inf, dtype=np.float64)
    idx = range(S) if seqs is None else seqs
    for i in idx:
        n = int(context_lens[i])
        Kc, Vc = gather_context(key_cache, value_cache, block_tables[i], n, block_size)
        Kf, Vf = decode_values(Kc, dtype), decode_values(Vc, dtype)
        q = decode_values(query[i], dtype)
        for p in range(num_parts):
            lo, hi = p * partition_size, min((p + 1) * partition_size, n)
            if lo >= hi:
                continue
            o_parts[i, :, p], lse_parts[i, :, p] = attention_contiguous(q, Kf[lo:hi], Vf[lo:hi], scale)
    return o_parts, lse_parts


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Exact merge of partial softmax results along the partition axis.

    With M = max_p lse_p and w_p = exp(lse_p - M):
    out = sum_p w_p o_p / sum_p w_p and lse = M + ln sum_p w_p. Partitions with
    lse_p = -inf carry no weight; if every partition is empty, out = 0 and
    lse = -inf.
    o_parts: [..., P, d]; lse_parts: [..., P].
    """
    o = np.asarray(o_parts, dtype=np.float64)
    lp = np.asarray(lse_parts, dtype=np.float64)
    M = lp.max(axis=-1)
    empty = ~np.isfinite(M)
    Ms = np.where(empty, 0.0, M)
    w = np.where(np.isfinite(lp), np.exp(lp - Ms[..., None]), 0.0)
    wsum = w.sum(axis=-1)
    # Zero-weight partitions are skipped rather than multiplied, so arbitrary
    # contents there (NaN included) cannot leak.
    o_used = np.where(w[..., None] > 0, o, 0.0)
    num = (w[..., None] * o_used).sum(axis=-2)
    safe = np.where(empty, 1.0, wsum)
    out = np.where(empty[..., None], 0.0, num / safe[..., None])
    lse = np.where(empty, -np.inf, Ms + np.log(safe))
    return out, lse


def reshape_and_cache(key: np.ndarray, value: np.ndarray, key_cache: np.ndarray,
                      value_cache: np.ndarray, slot_mapping: np.ndarray, block_size: int = 16):
    """Scatter each token's K/V row into its slot; return new (key_cache, value_cache).

    Token t goes to physical block ``slot // block_size``, offset
    ``slot % block_size``. A negative slot marks a padding token and is
    skipped; so is a slot past the pool (reading: the pages never write one).
    The inputs are not modified.
    """
    kc = key_cache.copy()
    vc = value_cache.copy()
    total = kc.shape[0] * block_size
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= total:
            continue
        kc[slot // block_size, slot % block_size] = key[t]
        vc[slot // block_size, slot % block_size] = value[t]
    return kc, vc


def copy_blocks(key_cache: np.ndarray, value_cache: np.ndarray, block_mapping):
    """Whole-block copies for copy-on-write; return new (key_cache, value_cache).

    For each (source, destination) pair, in order, the destination block's K
    and V (all token rows, all kv heads) become the source block's: the GPU
    half of copy-on-write, which gives a writer a private copy of a block that
    others still read (llm-stack-book 7.3 "vLLM: Architecture,
    PagedAttention & Internals", section "Copy-on-write for shared blocks").
    A pair naming a block outside the pool is skipped (reading: the pages
    never name one). The inputs are not modified.
    """
    kc = key_cache.copy()
    vc = value_cache.copy()
    nb = kc.shape[0]
    for src, dst in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        if not (0 <= src < nb and 0 <= dst < nb):
            continue
        kc[dst] = kc[src]
        vc[dst] = vc[src]
    return kc, vc
