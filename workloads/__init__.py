"""Seeded synthetic inputs for paged decode attention.

This module only draws and lays out inputs: context lengths, block
placement, query/key/value values, the new-token slot mapping. It holds no
attention arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``paged_kv_cache_150_amd``) can consume the same arrays without sharing any
of the method's computation.

Workload shapes follow the pages' statement of the problem:

* the paged pool is ``[num_blocks, block_size, H_kv, d_h]`` per layer, blocks
  of 16 tokens handed out from a shuffled free list
  (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention & Internals",
  sections "PagedAttention in one paragraph" and "The free list and the block
  table");
* the new token of each sequence is written at
  ``slot = block_table[pos // bs] * bs + pos % bs`` with ``pos = n - 1``
  (same page, section "The forward step in detail");
* model heads follow the Llama-3-8B shape, 32 layers x 8 KV heads x 128
  (modernaiengineering.com lesson 13.15 "vLLM: High-Throughput Serving with
  PagedAttention", listing "paged_kv.py") and a 70B-like 64-query-head variant
  sharing one long prefix (same lesson, "How PagedAttention shares memory").
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import dataclasses
import math
import os

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)


@dataclass(frozen=True)
class PagedConfig:
    """One synthetic decode workload (one layer, one decode step)."""

    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    dtype: str  # "f32" or "bf16"
    ctx: tuple  # ("uniform", lo, hi) | ("normal", mean, std, lo, hi) | ("prefix", prefix_tokens, lo, hi)
    seed: int
    partition_size: int = 512
    description: str = ""
    kv_dtype: str = ""     # "" (caches in dtype) or "fp8" (E4M3 codes, bf16 query/out)
    k_scale: float = 1.0   # FP8 caches: value = code value * scale
    v_scale: float = 1.0

    @property
    def scale(self) -> float:
        # 1/sqrt(d_h), the scale the model contract passes to Attention(...)
        # (llm-stack-book 7.3, "Serving a model vLLM has never seen").
        return 1.0 / math.sqrt(self.head_size)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def kv_elem_bytes(self) -> int:
        return 1 if self.cache_dtype == "fp8" else self.elem_bytes

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads


CONFIGS: list[PagedConfig] = [
    PagedConfig(
        name="tiny_f32", num_seqs=4, num_heads=4, num_kv_heads=2, head_size=64,
        block_size=16, num_blocks=64, dtype="f32", ctx=("uniform", 1, 100), seed=0,
        partition_size=32,
        description="Tiny fp32: 4 seqs, H_q=4, H_kv=2, d_h=64, ctx U{1..100}, 64-block pool"),
    PagedConfig(
        name="llama3_8b_b64", num_seqs=64, num_heads=32, num_kv_heads=8, head_size=128,
        block_size=16, num_blocks=16384, dtype="bf16", ctx=("uniform", 512, 2048), seed=1,
        partition_size=512,
        description="Llama-3-8B-shaped decode layer: batch 64, ctx U{512..2048}, 16k-block pool"),
    PagedConfig(
        name="llama3_8b_b256", num_seqs=256, num_heads=32, num_kv_heads=8, head_size=128,
        block_size=16, num_blocks=32768, dtype="bf16", ctx=("normal", 1000.0, 200.0, 16, 4096),
        seed=2, partition_size=512,
        description="Llama-3-8B-shaped decode: batch 256, ctx N(1000,200) clipped [16,4096], "
                    "reshape_and_cache of 256 new tokens first"),
    PagedConfig(
        name="long_split", num_seqs=8, num_heads=32, num_kv_heads=8, head_size=128,
        block_size=16, num_blocks=32768, dtype="bf16", ctx=("uniform", 16384, 32768), seed=3,
        partition_size=512,
        description="Long-context split-K: batch 8, ctx U{16k..32k}, 512-token partitions"),
    PagedConfig(
        name="prefix_70b", num_seqs=128, num_heads=64, num_kv_heads=8, head_size=128,
        block_size=16, num_blocks=16384, dtype="bf16", ctx=("prefix", 1024, 64, 512), seed=4,
        partition_size=512,
        description="70B-shaped heads: 128 seqs share one 1024-token prefix + suffix U{64..512}"),
]

# Beyond the five workloads above: the batch-256 step with an FP8 (E4M3) KV
# cache. Codes are drawn directly (log-uniform magnitudes); with the scales
# below, keys and values span about 2^-12 .. 4.
_BASE_BY_NAME = {c.name: c for c in CONFIGS}

EXTRA_CONFIGS: list[PagedConfig] = [
    dataclasses.replace(_BASE_BY_NAME["llama3_8b_b256"], name="llama3_8b_b256_fp8", kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 64,
                        description="Batch-256 Llama-3-8B-shaped decode over an FP8 E4M3 KV cache "
                                    "(bf16 query/out, k_scale = v_scale = 1/64)"),
]

CONFIG_BY_NAME = {c.name: c for c in CONFIGS + EXTRA_CONFIGS}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_context_lens(cfg: PagedConfig, rng: np.random.Generator) -> np.ndarray:
    kind = cfg.ctx[0]
    if kind == "uniform":
        _, lo, hi = cfg.ctx
        n = rng.integers(lo, hi + 1, size=cfg.num_seqs)
    elif kind == "normal":
        _, mean, std, lo, hi = cfg.ctx
        n = np.clip(np.rint(rng.normal(mean, std, size=cfg.num_seqs)), lo, hi)
    elif kind == "prefix":
        _, prefix, lo, hi = cfg.ctx
        n = prefix + rng.integers(lo, hi + 1, size=cfg.num_seqs)
    else:
        raise ValueError(kind)
    return n.astype(np.int32)


def draw_context_lens(cfg: PagedConfig, seed: int | None = None) -> np.ndarray:
    """The context lengths make_inputs() would draw (its first draw), without the rest."""
    return _draw_context_lens(cfg, np.random.default_rng(cfg.seed if seed is None else seed))


_CHUNK = 1 << 22  # elements per independent sub-stream of a large draw


def _values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) values of ``shape``: float32, or bfloat16 bits (RNE) for ``bf16``.

    One seed is drawn from ``rng``; the array is then filled in fixed chunks of
    2^22 elements, each from its own child stream of that seed
    (numpy SeedSequence.spawn), so the result does not depend on how many
    threads fill it.
    """
    n = int(np.prod(shape))
    seed = int(rng.integers(0, 2 ** 63))
    kids = np.random.SeedSequence(seed).spawn(max(1, -(-n // _CHUNK)))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = np.random.default_rng(kids[i]).standard_normal(size=hi - lo, dtype=np.float32)
        out[lo:hi] = x if dtype == "f32" else f32_to_bf16_bits(x)

    if len(kids) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(len(kids))))
    return out.reshape(shape)


def _codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Random FP8 E4M3 codes: uniform sign and mantissa, exponent field uniform
    in 1..14 (never NaN), i.e. log-uniform magnitudes 2^-6 .. 240. Drawn the
    same chunked way as _values."""
    n = int(np.prod(shape))
    seed = int(rng.integers(0, 2 ** 63))
    kids = np.random.SeedSequence(seed).spawn(max(1, -(-n // _CHUNK)))
    out = np.empty(n, dtype=np.uint8)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        u = np.random.default_rng(kids[i]).integers(0, 1 << 16, size=hi - lo, dtype=np.uint32)
        out[lo:hi] = ((u & 1) << 7 | (1 + (u >> 4) % 14) << 3 | (u >> 1) & 7).astype(np.uint8)

    if len(kids) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(len(kids))))
    return out.reshape(shape)


FP8_NAN_CODE = np.uint8(0x7F)


def poison_value(dtype: str):
    if dtype == "fp8":
        return FP8_NAN_CODE
    return np.float32(np.nan) if dtype == "f32" else BF16_NAN_BITS


def storage_dtype(dtype: str):
    if dtype == "fp8":
        return np.uint8
    return np.float32 if dtype == "f32" else np.uint16


@dataclass
class PagedInputs:
    """Host arrays for one workload.

    Caches are stored as float32 (``f32``) or as raw bfloat16 bits in uint16
    (``bf16``). ``key_cache``/``value_cache`` hold the full context, including
    the new token at position ``n-1``; ``new_key``/``new_value`` are that
    token's rows and ``slot_mapping`` its flat slot, so the state *before*
    reshape_and_cache is the pool with those slots overwritten by poison.
    """

    cfg: PagedConfig
    context_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray      # int32 [S, MB], padded with -1
    query: np.ndarray             # [S, H_q, d_h]
    key_cache: np.ndarray         # [NB, bs, H_kv, d_h]
    value_cache: np.ndarray       # [NB, bs, H_kv, d_h]
    new_key: np.ndarray           # [S, H_kv, d_h]
    new_value: np.ndarray         # [S, H_kv, d_h]
    slot_mapping: np.ndarray      # int64 [S]
    referenced_blocks: np.ndarray  # int64 [n_ref], physical ids in allocation order
    shared_prefix_blocks: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0


def make_inputs(cfg: PagedConfig, mode: str = "parity", seed: int | None = None,
                context_lens: np.ndarray | None = None) -> PagedInputs:
    """Draw one workload.

    Draw order from one PCG64 stream: context lengths, block placement (a
    permutation of the free list handed out in logical order), query, K blocks,
    V blocks. ``mode="parity"`` fills every slot that no sequence owns (tails of
    last blocks, unreferenced blocks) with NaN so that a stray read shows up in
    the output; ``mode="perf"`` leaves unreferenced blocks zero.
    ``context_lens`` optionally overrides the drawn lengths (same draw order).
    """
    if mode not in ("parity", "perf"):
        raise ValueError(mode)
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    S, bs = cfg.num_seqs, cfg.block_size
    n = _draw_context_lens(cfg, rng)
    if context_lens is not None:
        n = np.asarray(context_lens, dtype=np.int32).copy()
        S = n.shape[0]
    nblk = (n.astype(np.int64) + bs - 1) // bs

    prefix_blocks = 0
    if cfg.ctx[0] == "prefix":
        prefix_blocks = cfg.ctx[1] // bs
    private = nblk - prefix_blocks
    total = int(prefix_blocks + private.sum())
    if total > cfg.num_blocks:
        raise ValueError(f"{cfg.name}: needs {total} blocks, pool has {cfg.num_blocks}")

    free = rng.permutation(cfg.num_blocks)
    mb = int(max(1, nblk.max() if S else 1))
    tables = np.full((S, mb), -1, dtype=np.int32)
    cursor = 0
    shared = free[cursor:cursor + prefix_blocks]
    cursor += prefix_blocks
    alloc_order = [shared]
    for i in range(S):
        own = free[cursor:cursor + int(private[i])]
        cursor += int(private[i])
        tables[i, :prefix_blocks] = shared
        tables[i, prefix_blocks:nblk[i]] = own
        alloc_order.append(own)
    referenced = np.concatenate(alloc_order).astype(np.int64) if alloc_order else np.zeros(0, np.int64)

    Hq, Hkv, d = cfg.num_heads, cfg.num_kv_heads, cfg.head_size
    query = _values(rng, (S, Hq, d), cfg.dtype)

    cdt = cfg.cache_dtype
    sdt = storage_dtype(cdt)
    fill = poison_value(cdt) if mode == "parity" else sdt(0)
    caches = []
    for _ in range(2):  # K then V
        pool = np.empty((cfg.num_blocks, bs, Hkv, d), dtype=sdt)
        if mode == "parity":
            pool[...] = fill
        else:
            pool[...] = 0
        shape = (referenced.size, bs, Hkv, d)
        pool[referenced] = _codes(rng, shape) if cdt == "fp8" else _values(rng, shape, cfg.dtype)
        caches.append(pool)
    key_cache, value_cache = caches

    # Slots that no sequence owns (past n_i in its last block) are poisoned in
    # parity mode. Shared blocks are full by construction, so a tail is only
    # ever owned by one sequence.
    if mode == "parity":
        for i in range(S):
            if n[i] % bs and nblk[i] > 0:
                last = tables[i, nblk[i] - 1]
                key_cache[last, n[i] % bs:] = fill
                value_cache[last, n[i] % bs:] = fill

    # New token of each sequence sits at position n-1.
    pos = n.astype(np.int64) - 1
    slot = np.full(S, -1, dtype=np.int64)
    for i in range(S):
        if n[i] > 0:
            slot[i] = int(tables[i, pos[i] // bs]) * bs + int(pos[i] % bs)
    ok = slot >= 0
    if cdt == "fp8":
        # The new token's K/V arrive in the query's dtype and are quantized by
        # the write, so they are drawn here and the caches hold the state
        # before the write (their rows at the slots are overwritten by it).
        new_key = _values(rng, (S, Hkv, d), cfg.dtype)
        new_value = _values(rng, (S, Hkv, d), cfg.dtype)
    else:
        flat_k = key_cache.reshape(cfg.num_blocks * bs, Hkv, d)
        flat_v = value_cache.reshape(cfg.num_blocks * bs, Hkv, d)
        new_key = np.zeros((S, Hkv, d), dtype=sdt)
        new_value = np.zeros((S, Hkv, d), dtype=sdt)
        new_key[ok] = flat_k[slot[ok]]
        new_value[ok] = flat_v[slot[ok]]

    return PagedInputs(cfg=cfg, context_lens=n, block_tables=tables, query=query,
                       key_cache=key_cache, value_cache=value_cache, new_key=new_key,
                       new_value=new_value, slot_mapping=slot, referenced_blocks=referenced,
                       shared_prefix_blocks=prefix_blocks,
                       meta={"mode": mode, "seed": cfg.seed if seed is None else seed})


def caches_before_write(inp: PagedInputs):
    """Copies of the caches as they are before this step's new tokens are written.

    The new token of each sequence is the row at its slot; before the write that
    row holds poison (NaN), so a missing write shows up in the decode output.
    """
    cfg = inp.cfg
    rows = cfg.num_blocks * cfg.block_size
    kc = inp.key_cache.copy()
    vc = inp.value_cache.copy()
    ok = (inp.slot_mapping >= 0) & (inp.slot_mapping < rows)
    fill = poison_value(cfg.cache_dtype)
    kc.reshape(rows, cfg.num_kv_heads, cfg.head_size)[inp.slot_mapping[ok]] = fill
    vc.reshape(rows, cfg.num_kv_heads, cfg.head_size)[inp.slot_mapping[ok]] = fill
    return kc, vc


def contiguous_placement(inp: PagedInputs):
    """The same contexts with their blocks laid end to end from block 0, in
    allocation order (a shared prefix first, then each sequence's own blocks
    in logical order): returns (ids, tables, slots) where block k of the new
    pool is block ids[k] of the old one, and tables / slots are the workload's
    block tables and slot mapping in the new numbering (-1 kept)."""
    bs = inp.cfg.block_size
    ids = np.asarray(inp.referenced_blocks, dtype=np.int64)
    remap = np.full(inp.cfg.num_blocks, -1, dtype=np.int64)
    remap[ids] = np.arange(ids.size)
    bt = inp.block_tables
    tables = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    s = inp.slot_mapping
    ok = s >= 0
    slots = np.full_like(s, -1)
    slots[ok] = remap[s[ok] // bs] * bs + s[ok] % bs
    return ids, tables, slots


def reorder_multi_inputs(mq: "MultiQueryInputs", order: np.ndarray) -> "MultiQueryInputs":
    """The same multi-query step with its sequences listed in ``order``
    (sequence k of the result is sequence order[k] of ``mq``): tables, lengths,
    and each sequence's query rows, slots and new K/V rows move together; the
    caches are unchanged."""
    order = np.asarray(order, dtype=np.int64)
    loc = mq.query_start_loc
    rows = np.concatenate([np.arange(loc[i], loc[i + 1]) for i in order]).astype(np.int64) \
        if order.size else np.zeros(0, np.int64)
    qlens = mq.query_lens[order].astype(np.int32)
    new_loc = np.zeros(order.size + 1, np.int32)
    new_loc[1:] = np.cumsum(qlens)
    p = mq.paged
    paged = dataclasses.replace(p, context_lens=p.context_lens[order].copy(),
                                block_tables=p.block_tables[order].copy())
    return dataclasses.replace(mq, paged=paged, query_lens=qlens, query_start_loc=new_loc,
                               query=mq.query[rows].copy(), slot_mapping=mq.slot_mapping[rows].copy(),
                               new_key=mq.new_key[rows].copy(), new_value=mq.new_value[rows].copy())


def algorithmic_kv_bytes(cfg: PagedConfig, context_lens: np.ndarray) -> int:
    """K and V bytes one decode call must read: sum_i n_i * 2 * H_kv * d_h * b."""
    return int(np.asarray(context_lens, dtype=np.int64).sum()) * 2 * cfg.num_kv_heads * cfg.head_size * cfg.kv_elem_bytes


def unique_kv_bytes(inp: PagedInputs) -> int:
    """K and V bytes of distinct physical slots read (shared prefix blocks counted once)."""
    cfg = inp.cfg
    bs = cfg.block_size
    seen = set()
    total_tokens = 0
    for i in range(inp.context_lens.shape[0]):
        n = int(inp.context_lens[i])
        for j in range((n + bs - 1) // bs):
            b = int(inp.block_tables[i, j])
            used = min(bs, n - j * bs)
            key = b
            if key in seen:
                continue
            seen.add(key)
            total_tokens += used
    return total_tokens * 2 * cfg.num_kv_heads * cfg.head_size * cfg.kv_elem_bytes


# ---------------------------------------------------------------- several new tokens per sequence
@dataclass(frozen=True)
class MultiQueryConfig:
    """One step in which sequences may process more than one new token.

    ``base`` gives the head shape, pool and drawn context lengths (the stored
    tokens after the step, new ones included). ``new_tokens`` is
    ("fixed", q): every sequence has q new tokens (a speculative step verifying
    q - 1 draft tokens, llm-stack-book 7.3, "Speculative decoding support"), or
    ("chunk", m, c, n): the first m sequences run a c-token prompt chunk that
    ends at context length n, the others one decode token each (one forward
    pass mixing a prefill slice with decodes, same page, "Prefill, decode, and
    chunked prefill").
    """

    name: str
    base: PagedConfig
    new_tokens: tuple
    description: str = ""


MQ_CONFIGS: list[MultiQueryConfig] = [
    MultiQueryConfig(
        name="llama3_8b_b64_spec4", base=CONFIG_BY_NAME["llama3_8b_b64"], new_tokens=("fixed", 5),
        description="Speculative verify on the batch-64 Llama-3-8B-shaped decode: k = 4 draft tokens, "
                    "5 new positions per sequence, ctx U{512..2048}"),
    MultiQueryConfig(
        name="llama3_8b_b256_chunk1024", base=CONFIG_BY_NAME["llama3_8b_b256"], new_tokens=("chunk", 1, 1024, 2048),
        description="The batch-256 decode step with one sequence running a 1024-token prompt chunk "
                    "(tokens 1024..2047 of its prompt) in the same pass"),
    MultiQueryConfig(
        name="long_split_spec4", base=CONFIG_BY_NAME["long_split"], new_tokens=("fixed", 5),
        description="Speculative verify on the long-context batch: 8 sequences, ctx U{16k..32k}, "
                    "5 new positions each (few tiles over long contexts)"),
]

MQ_CONFIG_BY_NAME = {c.name: c for c in MQ_CONFIGS}


@dataclass
class MultiQueryInputs:
    """Host arrays of one multi-query step. ``paged`` holds the caches with every
    context complete (new tokens included), the tables and the lengths; the
    new tokens of sequence i are rows query_start_loc[i] .. query_start_loc[i+1]
    of ``query`` and positions n_i - q_i .. n_i - 1 of its context."""

    cfg: MultiQueryConfig
    paged: PagedInputs
    query_lens: np.ndarray        # int32 [S]
    query_start_loc: np.ndarray   # int32 [S + 1]
    query: np.ndarray             # [T, H_q, d_h]
    slot_mapping: np.ndarray      # int64 [T], -1 for a token with no position
    new_key: np.ndarray           # [T, H_kv, d_h] (rows of the caches at the slots)
    new_value: np.ndarray

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])


def multi_lengths(cfg: MultiQueryConfig, seed: int | None = None, context_lens: np.ndarray | None = None,
                  query_lens: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Context lengths n (new tokens included) and new-token counts q of one
    multi-query step, as ``new_tokens`` says (or as given)."""
    base = cfg.base
    s = base.seed if seed is None else seed
    n = draw_context_lens(base, s) if context_lens is None else np.asarray(context_lens, np.int32).copy()
    S = n.shape[0]
    kind = cfg.new_tokens[0]
    if query_lens is not None:
        q = np.asarray(query_lens, np.int32).copy()
    elif kind == "fixed":
        q = np.full(S, cfg.new_tokens[1], np.int32)
        n = np.maximum(n, q)
    elif kind == "chunk":
        _, m, c, ctx = cfg.new_tokens
        q = np.ones(S, np.int32)
        q[:m] = c
        if context_lens is None:
            n[:m] = ctx
    else:
        raise ValueError(kind)
    return n, q


def make_multi_inputs(cfg: MultiQueryConfig, mode: str = "parity", seed: int | None = None,
                      context_lens: np.ndarray | None = None, query_lens: np.ndarray | None = None
                      ) -> MultiQueryInputs:
    """Draw one multi-query step: the base workload's inputs (make_inputs, same
    draws) with the lengths adjusted as ``new_tokens`` says, then the new
    tokens' queries from a second stream. ``context_lens``/``query_lens``
    override the lengths."""
    base = cfg.base
    s = base.seed if seed is None else seed
    n, q = multi_lengths(cfg, s, context_lens, query_lens)
    S = n.shape[0]
    inp = make_inputs(base, mode, seed=s, context_lens=n)
    loc = np.concatenate([[0], np.cumsum(q, dtype=np.int64)]).astype(np.int32)
    T = int(loc[-1])
    rng = np.random.default_rng([s, 101])
    query = _values(rng, (T, base.num_heads, base.head_size), base.dtype)
    bs = base.block_size
    slots = np.full(T, -1, np.int64)
    for i in range(S):
        for j in range(int(q[i])):
            p = int(n[i]) - int(q[i]) + j
            if p >= 0:
                slots[loc[i] + j] = int(inp.block_tables[i, p // bs]) * bs + p % bs
    rows = base.num_blocks * bs
    ok = slots >= 0
    shape = (T, base.num_kv_heads, base.head_size)
    new_key = np.zeros(shape, inp.key_cache.dtype)
    new_value = np.zeros(shape, inp.value_cache.dtype)
    new_key[ok] = inp.key_cache.reshape(rows, *shape[1:])[slots[ok]]
    new_value[ok] = inp.value_cache.reshape(rows, *shape[1:])[slots[ok]]
    return MultiQueryInputs(cfg=cfg, paged=inp, query_lens=q, query_start_loc=loc, query=query,
                            slot_mapping=slots, new_key=new_key, new_value=new_value)


def multi_caches_before_write(mq: MultiQueryInputs):
    """The caches before this step's new tokens are written: their rows poisoned."""
    base = mq.cfg.base
    rows = base.num_blocks * base.block_size
    kc, vc = mq.paged.key_cache.copy(), mq.paged.value_cache.copy()
    ok = mq.slot_mapping >= 0
    fill = poison_value(base.cache_dtype)
    kc.reshape(rows, base.num_kv_heads, base.head_size)[mq.slot_mapping[ok]] = fill
    vc.reshape(rows, base.num_kv_heads, base.head_size)[mq.slot_mapping[ok]] = fill
    return kc, vc


def multi_query_flops(mq: MultiQueryInputs) -> int:
    """Multiply-adds x 2 of the step's attention: for each new token and query
    head, 2 d_h flops for its score and 2 d_h for its P*V term per visible key."""
    base = mq.cfg.base
    vis = 0
    for i in range(mq.query_lens.shape[0]):
        n, q = int(mq.paged.context_lens[i]), int(mq.query_lens[i])
        first = max(n - q + 1, 0)          # visible keys of the first new token
        last = max(n, 0)
        k = max(0, last - first + 1)       # tokens with at least one visible key
        vis += (first + last) * k // 2
    return 4 * base.num_heads * base.head_size * vis


def small_case(name: str, num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
               dtype: str, ctx: tuple, seed: int, num_blocks: int, partition_size: int = 64,
               kv_dtype: str = "", k_scale: float = 1.0, v_scale: float = 1.0) -> PagedConfig:
    """A small ad-hoc config for parity sweeps (same generator, different shape)."""
    return PagedConfig(name=name, num_seqs=num_seqs, num_heads=num_heads,
                       num_kv_heads=num_kv_heads, head_size=head_size, block_size=16,
                       num_blocks=num_blocks, dtype=dtype, ctx=ctx, seed=seed,
                       partition_size=partition_size, description="ad-hoc parity case",
                       kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale)
