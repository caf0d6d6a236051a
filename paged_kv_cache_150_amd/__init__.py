"""Paged KV-cache decode attention for AMD MI355X (gfx950).

Thin Python binding over ``libpa.so`` (declared in ``include/pa.h``). Each
function has the name of the C entry point it calls and only marshals
arguments: it checks that tensors live on the GPU, are contiguous and agree in
shape (the C side receives raw pointers and cannot), then passes device
pointers and the current HIP stream. Every step of the computation runs in the
library's HIP kernels; there is no fallback. If ``libpa.so`` has not been built
the first call raises.

PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "PA_DTYPE_F32", "PA_DTYPE_BF16", "PaError", "library_path", "load_library", "prepared",
    "pa_reshape_and_cache", "pa_reshape_and_cache_fp8", "pa_copy_blocks", "pa_decode", "pa_decode_fp8",
    "pa_reshape_and_decode", "pa_reshape_and_decode_fp8",
    "pa_multi_query", "pa_multi_query_fp8", "pa_multi_query_split_workspace_bytes", "pa_multi_query_split",
    "pa_multi_query_split_partition_size",
    "pa_decode_prefix_workspace_bytes", "pa_decode_prefix",
    "pa_decode_split_workspace_bytes", "pa_decode_split", "pa_decode_split_part_tokens",
    "pa_decode_split_noalloc", "PA_DECODE_SPLIT_NOALLOC_MAX_BYTES", "pa_stream_read", "pa_stream_kv",
    "pa_merge_partitions", "pa_status_string", "pa_set_option", "pa_get_option", "options",
    "PA_OPT_TILE_WAVES", "PA_OPT_TILE_COLUMNS", "PA_OPT_SPLIT_CUT", "PA_OPT_SPLIT_PART_FACTOR", "PA_OPT_MERGE_ROWS",
]

PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
BLOCK_SIZE = 16

# Kernel-choice options (pa_option in include/pa.h); 0 is the default choice.
PA_OPT_TILE_WAVES = 0         # 0, 4 or 8
PA_OPT_TILE_COLUMNS = 1       # 0, 16 or 32
PA_OPT_SPLIT_CUT = 2          # 0, 1 (partitions) or 2 (pieces)
PA_OPT_SPLIT_PART_FACTOR = 3  # 0 or k >= 1
PA_OPT_MERGE_ROWS = 4         # 0, 1, 2 or 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {pa_status_string(status)} (status {status})")


def library_path() -> str:
    """The in-tree libpa.so, or the file PA_LIBRARY names (the host-sanitizer
    build of the tests uses this)."""
    return os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpa.so")


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_150_amd.build` "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    c_int, c_i32, c_i64, c_f, c_p, c_sz = (ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                          ctypes.c_void_p, ctypes.c_size_t)
    lib.pa_reshape_and_cache.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_p]
    lib.pa_reshape_and_cache.restype = c_int
    lib.pa_reshape_and_cache_fp8.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32,
                                             c_f, c_f, c_p]
    lib.pa_reshape_and_cache_fp8.restype = c_int
    lib.pa_decode_fp8.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i64, c_i32,
                                  c_f, c_f, c_f, c_i32, c_p, c_p, c_p]
    lib.pa_decode_fp8.restype = c_int
    lib.pa_copy_blocks.argtypes = [c_p, c_p, c_p, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_p]
    lib.pa_copy_blocks.restype = c_int
    lib.pa_decode.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i64, c_i32,
                              c_f, c_i32, c_p, c_p, c_p]
    lib.pa_decode.restype = c_int
    lib.pa_multi_query.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                   c_i64, c_i32, c_f, c_i32, c_p, c_p]
    lib.pa_multi_query.restype = c_int
    lib.pa_reshape_and_decode.argtypes = [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32,
                                          c_i32, c_i64, c_i32, c_f, c_i32, c_p, c_p, c_p]
    lib.pa_reshape_and_decode.restype = c_int
    lib.pa_reshape_and_decode_fp8.argtypes = [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32,
                                              c_i32, c_i32, c_i64, c_i32, c_f, c_f, c_f, c_i32, c_p, c_p, c_p]
    lib.pa_reshape_and_decode_fp8.restype = c_int
    lib.pa_set_option.argtypes = [c_int, c_int]
    lib.pa_set_option.restype = c_int
    lib.pa_get_option.argtypes = [c_int]
    lib.pa_get_option.restype = c_int
    lib.pa_decode_split_part_tokens.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]
    lib.pa_decode_split_part_tokens.restype = c_i32
    lib.pa_multi_query_fp8.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                       c_i64, c_i32, c_f, c_f, c_f, c_i32, c_p, c_p]
    lib.pa_multi_query_fp8.restype = c_int
    lib.pa_decode_prefix_workspace_bytes.argtypes = [c_i32, c_i32, c_i32]
    lib.pa_decode_prefix_workspace_bytes.restype = c_sz
    lib.pa_decode_prefix.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i64, c_i32,
                                     c_f, c_i32, c_i32, c_p, c_sz, c_p, c_p, c_p]
    lib.pa_decode_prefix.restype = c_int
    lib.pa_multi_query_split_workspace_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32]
    lib.pa_multi_query_split_workspace_bytes.restype = c_sz
    lib.pa_multi_query_split_partition_size.argtypes = [c_i32] * 7
    lib.pa_multi_query_split_partition_size.restype = c_i32
    lib.pa_multi_query_split.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                         c_i64, c_i32, c_f, c_i32, c_i32, c_i32, c_p, c_sz, c_p, c_p]
    lib.pa_multi_query_split.restype = c_int
    lib.pa_decode_split_workspace_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32]
    lib.pa_decode_split_workspace_bytes.restype = c_sz
    lib.pa_decode_split.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i64,
                                    c_i32, c_f, c_i32, c_i32, c_i32, c_p, c_sz, c_p, c_p]
    lib.pa_decode_split.restype = c_int
    lib.pa_decode_split_noalloc.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i64,
                                            c_i32, c_f, c_i32, c_i32, c_i32, c_p, c_p]
    lib.pa_decode_split_noalloc.restype = c_int
    lib.pa_stream_read.argtypes = [c_p, c_sz, c_p, c_p]
    lib.pa_stream_read.restype = c_int
    lib.pa_stream_kv.argtypes = [c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i64, c_i32, c_i32, c_p, c_p, c_p]
    lib.pa_stream_kv.restype = c_int
    lib.pa_merge_partitions.argtypes = [c_p, c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_p]
    lib.pa_merge_partitions.restype = c_int
    lib.pa_status_string.argtypes = [c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def pa_status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def pa_set_option(option: int, value: int) -> None:
    """Force a kernel choice process-wide (see pa_option in include/pa.h); 0 restores the default."""
    _check(load_library().pa_set_option(int(option), int(value)), "pa_set_option")


def pa_get_option(option: int) -> int:
    v = int(load_library().pa_get_option(int(option)))
    if v < 0:
        raise ValueError(f"unknown option {option}")
    return v


class options:
    """Context manager: ``with options({PA_OPT_SPLIT_CUT: 2}): ...`` sets the
    given options and restores their previous values on exit."""

    def __init__(self, values: dict):
        self._values = dict(values)
        self._saved = {}

    def __enter__(self):
        for k, v in self._values.items():
            self._saved[k] = pa_get_option(k)
            pa_set_option(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self._saved.items():
            pa_set_option(k, v)
        return False


# ------------------------------------------------------------------ marshalling helpers
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


_capture = threading.local()


def _invoke(fn, where: str, *args) -> None:
    """One library call with its status checked, or, inside prepared(), the
    call recorded for replay."""
    rec = getattr(_capture, "calls", None)
    if rec is not None:
        rec.append((fn, args, where))
        return
    _check(fn(*args), where)


def prepared(fn, *args, **kwargs):
    """Validate the arguments of binding function ``fn`` once and return a
    zero-argument callable that repeats exactly the same library call(s)
    (same tensors, sizes and stream) with only the ctypes call per launch.
    For launch loops where the per-call checks would cost more than the
    kernel; the tensors must stay alive and unchanged in shape."""
    _capture.calls = []
    try:
        fn(*args, **kwargs)
        calls = _capture.calls
    finally:
        _capture.calls = None

    def run():
        for f, a, where in calls:
            _check(f(*a), where)
    return run


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PaError(status, where)


def _cache_dims(key_cache: torch.Tensor, value_cache: torch.Tensor):
    if key_cache.shape != value_cache.shape or key_cache.dtype != value_cache.dtype:
        raise ValueError("key_cache and value_cache must have the same shape and dtype")
    if key_cache.dim() != 4:
        raise ValueError("caches must be [num_blocks, block_size, num_kv_heads, head_size]")
    return tuple(int(x) for x in key_cache.shape)


# ------------------------------------------------------------------ entry points
def pa_reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                         value_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Write key[t], value[t] into cache slot slot_mapping[t] (negative slot: skipped)."""
    NB, bs, Hkv, d = _cache_dims(key_cache, value_cache)
    if key.shape != value.shape or key.dim() != 3 or tuple(key.shape[1:]) != (Hkv, d):
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_size] matching the cache")
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype:
        raise TypeError("key/value dtype must match the cache dtype")
    T = int(key.shape[0])
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    lib = load_library()
    _invoke(lib.pa_reshape_and_cache, "pa_reshape_and_cache", _dev(key, "key"), _dev(value, "value"),
            _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            _dev(slot_mapping, "slot_mapping", torch.int64, 1), T, NB, bs, Hkv, d, _dtype_code(key_cache),
            _stream(stream))


def pa_copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, block_mapping: torch.Tensor,
                   stream=None) -> None:
    """Copy whole blocks: block_mapping int64 [num_pairs, 2] of (source, destination)."""
    NB, bs, Hkv, d = _cache_dims(key_cache, value_cache)
    if block_mapping.dim() != 2 or int(block_mapping.shape[1]) != 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    lib = load_library()
    _invoke(lib.pa_copy_blocks, "pa_copy_blocks", _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            _dev(block_mapping, "block_mapping", torch.int64, 2), int(block_mapping.shape[0]), NB, bs, Hkv, d,
            _dtype_code(key_cache), _stream(stream))


def _decode_common(out, query, key_cache, value_cache, block_tables, context_lens, lse_out, fp8=False):
    NB, bs, Hkv, d = _cache_dims(key_cache, value_cache)
    if query.dim() != 3 or int(query.shape[2]) != d:
        raise ValueError("query must be [num_seqs, num_heads, head_size]")
    S, Hq = int(query.shape[0]), int(query.shape[1])
    if fp8:
        if key_cache.dtype != torch.uint8:
            raise TypeError("FP8 caches are uint8 tensors of E4M3 codes")
        if out.shape != query.shape or out.dtype != query.dtype:
            raise ValueError("out must match query's shape and dtype")
    elif out.shape != query.shape or out.dtype != query.dtype or query.dtype != key_cache.dtype:
        raise ValueError("out must match query's shape; query, out and caches share one dtype")
    if block_tables.dim() != 2 or int(block_tables.shape[0]) != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if context_lens.shape != (S,):
        raise ValueError("context_lens must be [num_seqs]")
    lse_ptr = None
    if lse_out is not None:
        if lse_out.shape != (S, Hq):
            raise ValueError("lse_out must be [num_seqs, num_heads]")
        lse_ptr = _dev(lse_out, "lse_out", torch.float32)
    ptrs = dict(out=_dev(out, "out"), query=_dev(query, "query"), kc=_dev(key_cache, "key_cache"),
                vc=_dev(value_cache, "value_cache"),
                bt=_dev(block_tables, "block_tables", torch.int32, 2),
                cl=_dev(context_lens, "context_lens", torch.int32, 1), lse=lse_ptr)
    return ptrs, (S, Hq, Hkv, d, NB, bs, int(block_tables.shape[1]))


def pa_decode(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
              block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
              lse_out: torch.Tensor | None = None, seq_order: torch.Tensor | None = None,
              stream=None) -> None:
    """One-pass paged decode attention into ``out`` (optionally ln-sum-exp into ``lse_out``).

    ``seq_order`` (int32 [num_seqs], a permutation) is a schedule hint: the order
    in which sequences are handed out, e.g. longest first. Results do not depend on it.
    """
    p, (S, Hq, Hkv, d, NB, bs, MB) = _decode_common(out, query, key_cache, value_cache, block_tables,
                                                   context_lens, lse_out)
    order_ptr = None
    if seq_order is not None:
        if seq_order.shape != (S,):
            raise ValueError("seq_order must be [num_seqs]")
        order_ptr = _dev(seq_order, "seq_order", torch.int32, 1)
    lib = load_library()
    _invoke(lib.pa_decode, "pa_decode", p["out"], p["query"], p["kc"], p["vc"], p["bt"], MB, p["cl"], S, Hq, Hkv, d,
            NB, bs, float(scale), _dtype_code(query), p["lse"], order_ptr, _stream(stream))


def _multi_common(out, query, key_cache, value_cache, block_tables, context_lens, query_start_loc, lse_out,
                  fp8=False):
    NB, bs, Hkv, d = _cache_dims(key_cache, value_cache)
    if query.dim() != 3 or int(query.shape[2]) != d:
        raise ValueError("query must be [num_tokens, num_heads, head_size]")
    T, Hq = int(query.shape[0]), int(query.shape[1])
    if fp8:
        if key_cache.dtype != torch.uint8:
            raise TypeError("FP8 caches are uint8 tensors of E4M3 codes")
        if out.shape != query.shape or out.dtype != query.dtype:
            raise ValueError("out must match query's shape and dtype")
    elif out.shape != query.shape or out.dtype != query.dtype or query.dtype != key_cache.dtype:
        raise ValueError("out must match query's shape; query, out and caches share one dtype")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    S = int(block_tables.shape[0])
    if context_lens.shape != (S,) or query_start_loc.shape != (S + 1,):
        raise ValueError("context_lens must be [num_seqs] and query_start_loc [num_seqs + 1]")
    lse_ptr = None
    if lse_out is not None:
        if lse_out.shape != (T, Hq):
            raise ValueError("lse_out must be [num_tokens, num_heads]")
        lse_ptr = _dev(lse_out, "lse_out", torch.float32)
    ptrs = (_dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            _dev(block_tables, "block_tables", torch.int32, 2), int(block_tables.shape[1]),
            _dev(context_lens, "context_lens", torch.int32, 1),
            _dev(query_start_loc, "query_start_loc", torch.int32, 1), S, T, Hq, Hkv, d, NB, bs)
    return ptrs, lse_ptr


def pa_multi_query(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                   scale: float, lse_out: torch.Tensor | None = None, stream=None) -> None:
    """Paged attention for several new tokens per sequence (prompt chunks, speculative positions).

    ``query``/``out`` are [num_tokens, num_heads, head_size]; sequence i's new
    tokens are rows ``query_start_loc[i] .. query_start_loc[i+1]`` (int32
    [num_seqs + 1]) and are the last of its ``context_lens[i]`` stored tokens.
    """
    ptrs, lse_ptr = _multi_common(out, query, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                                  lse_out)
    lib = load_library()
    _invoke(lib.pa_multi_query, "pa_multi_query", *ptrs, float(scale), _dtype_code(query), lse_ptr, _stream(stream))


def pa_multi_query_fp8(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                       block_tables: torch.Tensor, context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                       scale: float, k_scale: float, v_scale: float, lse_out: torch.Tensor | None = None,
                       stream=None) -> None:
    """pa_multi_query over FP8 (E4M3 code) caches with scales k_scale, v_scale; bf16 query/out."""
    ptrs, lse_ptr = _multi_common(out, query, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                                  lse_out, fp8=True)
    lib = load_library()
    _invoke(lib.pa_multi_query_fp8, "pa_multi_query_fp8", *ptrs, float(scale), float(k_scale), float(v_scale),
            _dtype_code(query), lse_ptr, _stream(stream))


def pa_multi_query_split_workspace_bytes(num_tokens: int, num_heads: int, head_size: int, max_context_len: int,
                                         partition_size: int) -> int:
    return int(load_library().pa_multi_query_split_workspace_bytes(num_tokens, num_heads, head_size,
                                                                   max_context_len, partition_size))


def pa_multi_query_split_partition_size(num_seqs: int, num_tokens: int, num_heads: int, num_kv_heads: int,
                                        head_size: int, max_context_len: int, dtype: int = PA_DTYPE_BF16) -> int:
    """Partition length for pa_multi_query_split, or 0 when pa_multi_query fills the GPU by itself."""
    return int(load_library().pa_multi_query_split_partition_size(num_seqs, num_tokens, num_heads, num_kv_heads,
                                                                  head_size, dtype, max_context_len))


def pa_multi_query_split(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                         scale: float, max_context_len: int, partition_size: int, workspace: torch.Tensor,
                         lse_out: torch.Tensor | None = None, stream=None) -> None:
    """pa_multi_query with every context cut into partition_size-token partitions and merged by
    log-sum-exp; ``workspace`` is a uint8 GPU tensor of pa_multi_query_split_workspace_bytes bytes."""
    ptrs, lse_ptr = _multi_common(out, query, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                                  lse_out)
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    _invoke(lib.pa_multi_query_split, "pa_multi_query_split", *ptrs, float(scale), _dtype_code(query),
            int(max_context_len), int(partition_size), ws, nbytes, lse_ptr, _stream(stream))


def pa_decode_split_part_tokens(num_seqs: int, num_heads: int, num_kv_heads: int, max_context_len: int,
                                partition_size: int, dtype: int = PA_DTYPE_BF16) -> int:
    """Partition length of pa_decode_split's partition cut for these arguments, or 0 for its pieces cut."""
    r = load_library().pa_decode_split_part_tokens(num_seqs, num_heads, num_kv_heads, max_context_len,
                                                   partition_size, dtype)
    if r < 0:
        raise ValueError("invalid split arguments")
    return int(r)


def pa_decode_prefix_workspace_bytes(num_seqs: int, num_heads: int, head_size: int) -> int:
    return int(load_library().pa_decode_prefix_workspace_bytes(num_seqs, num_heads, head_size))


def pa_decode_prefix(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                     block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, prefix_blocks: int,
                     workspace: torch.Tensor, lse_out: torch.Tensor | None = None,
                     seq_order: torch.Tensor | None = None, stream=None) -> None:
    """pa_decode for sequences whose first ``prefix_blocks`` block-table entries
    are shared (equal to row 0's): the shared blocks are read once for the batch."""
    p, (S, Hq, Hkv, d, NB, bs, MB) = _decode_common(out, query, key_cache, value_cache, block_tables,
                                                   context_lens, lse_out)
    order_ptr = None
    if seq_order is not None:
        if seq_order.shape != (S,):
            raise ValueError("seq_order must be [num_seqs]")
        order_ptr = _dev(seq_order, "seq_order", torch.int32, 1)
    ws = _dev(workspace, "workspace")
    lib = load_library()
    _invoke(lib.pa_decode_prefix, "pa_decode_prefix", p["out"], p["query"], p["kc"], p["vc"], p["bt"], MB, p["cl"],
            S, Hq, Hkv, d, NB, bs, float(scale), _dtype_code(query), int(prefix_blocks), ws,
            workspace.numel() * workspace.element_size(), p["lse"], order_ptr, _stream(stream))


def pa_reshape_and_decode(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                          slot_mapping: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                          block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                          lse_out: torch.Tensor | None = None, seq_order: torch.Tensor | None = None,
                          stream=None) -> None:
    """One decode step in one launch: write sequence i's new key[i]/value[i] to
    slot_mapping[i] (the slot of its last position), then pa_decode."""
    p, (S, Hq, Hkv, d, NB, bs, MB) = _decode_common(out, query, key_cache, value_cache, block_tables,
                                                   context_lens, lse_out)
    if key.shape != (S, Hkv, d) or value.shape != (S, Hkv, d) or key.dtype != key_cache.dtype \
            or value.dtype != key_cache.dtype:
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_size] in the cache dtype")
    if slot_mapping.shape != (S,):
        raise ValueError("slot_mapping must be [num_seqs]")
    order_ptr = None
    if seq_order is not None:
        if seq_order.shape != (S,):
            raise ValueError("seq_order must be [num_seqs]")
        order_ptr = _dev(seq_order, "seq_order", torch.int32, 1)
    lib = load_library()
    _invoke(lib.pa_reshape_and_decode, "pa_reshape_and_decode", p["out"], p["query"], _dev(key, "key"),
            _dev(value, "value"), _dev(slot_mapping, "slot_mapping", torch.int64, 1), p["kc"], p["vc"], p["bt"],
            MB, p["cl"], S, Hq, Hkv, d, NB, bs, float(scale), _dtype_code(query), p["lse"], order_ptr,
            _stream(stream))


def pa_reshape_and_decode_fp8(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                              slot_mapping: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                              block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, k_scale: float,
                              v_scale: float, lse_out: torch.Tensor | None = None,
                              seq_order: torch.Tensor | None = None, stream=None) -> None:
    """One FP8 decode step in one launch: quantize sequence i's new bf16
    key[i]/value[i] into slot_mapping[i] of the uint8 (E4M3) caches, then
    pa_decode_fp8."""
    p, (S, Hq, Hkv, d, NB, bs, MB) = _decode_common(out, query, key_cache, value_cache, block_tables,
                                                   context_lens, lse_out, fp8=True)
    if key.shape != (S, Hkv, d) or value.shape != (S, Hkv, d) or key.dtype != query.dtype \
            or value.dtype != query.dtype:
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_size] in the query dtype")
    if slot_mapping.shape != (S,):
        raise ValueError("slot_mapping must be [num_seqs]")
    order_ptr = None
    if seq_order is not None:
        if seq_order.shape != (S,):
            raise ValueError("seq_order must be [num_seqs]")
        order_ptr = _dev(seq_order, "seq_order", torch.int32, 1)
    lib = load_library()
    _invoke(lib.pa_reshape_and_decode_fp8, "pa_reshape_and_decode_fp8", p["out"], p["query"], _dev(key, "key"),
            _dev(value, "value"), _dev(slot_mapping, "slot_mapping", torch.int64, 1), p["kc"], p["vc"], p["bt"],
            MB, p["cl"], S, Hq, Hkv, d, NB, bs, float(scale), float(k_scale), float(v_scale), _dtype_code(query),
            p["lse"], order_ptr, _stream(stream))


def pa_reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                             value_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float, v_scale: float,
                             stream=None) -> None:
    """Quantize key[t], value[t] to E4M3 codes (uint8 caches) at slot_mapping[t]."""
    NB, bs, Hkv, d = _cache_dims(key_cache, value_cache)
    if key_cache.dtype != torch.uint8:
        raise TypeError("FP8 caches are uint8 tensors of E4M3 codes")
    if key.shape != value.shape or key.dim() != 3 or tuple(key.shape[1:]) != (Hkv, d):
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_size] matching the cache")
    T = int(key.shape[0])
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    lib = load_library()
    _invoke(lib.pa_reshape_and_cache_fp8, "pa_reshape_and_cache_fp8", _dev(key, "key"), _dev(value, "value"),
            _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            _dev(slot_mapping, "slot_mapping", torch.int64, 1), T, NB, bs, Hkv, d, _dtype_code(key), float(k_scale),
            float(v_scale), _stream(stream))


def pa_decode_fp8(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                  block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, k_scale: float,
                  v_scale: float, lse_out: torch.Tensor | None = None, seq_order: torch.Tensor | None = None,
                  stream=None) -> None:
    """pa_decode over FP8 (E4M3 code) caches with scales k_scale, v_scale; bf16 query/out."""
    p, (S, Hq, Hkv, d, NB, bs, MB) = _decode_common(out, query, key_cache, value_cache, block_tables,
                                                   context_lens, lse_out, fp8=True)
    order_ptr = None
    if seq_order is not None:
        if seq_order.shape != (S,):
            raise ValueError("seq_order must be [num_seqs]")
        order_ptr = _dev(seq_order, "seq_order", torch.int32, 1)
    lib = load_library()
    _invoke(lib.pa_decode_fp8, "pa_decode_fp8", p["out"], p["query"], p["kc"], p["vc"], p["bt"], MB, p["cl"], S, Hq,
            Hkv, d, NB, bs, float(scale), float(k_scale), float(v_scale), _dtype_code(query), p["lse"], order_ptr,
            _stream(stream))


def pa_decode_split_workspace_bytes(num_seqs: int, num_heads: int, head_size: int, max_context_len: int,
                                    partition_size: int) -> int:
    return int(load_library().pa_decode_split_workspace_bytes(num_seqs, num_heads, head_size,
                                                              max_context_len, partition_size))


def pa_decode_split(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                    value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                    scale: float, max_context_len: int, partition_size: int, workspace: torch.Tensor,
                    lse_out: torch.Tensor | None = None, stream=None) -> None:
    """Partitioned paged decode + log-sum-exp merge; ``workspace`` is a uint8 GPU tensor."""
    p, (S, Hq, Hkv, d, NB, bs, MB) = _decode_common(out, query, key_cache, value_cache, block_tables,
                                                   context_lens, lse_out)
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    _invoke(lib.pa_decode_split, "pa_decode_split", p["out"], p["query"], p["kc"], p["vc"], p["bt"], MB, p["cl"], S,
            Hq, Hkv, d, NB, bs, float(scale), _dtype_code(query), int(max_context_len), int(partition_size), ws,
            nbytes, p["lse"], _stream(stream))


PA_DECODE_SPLIT_NOALLOC_MAX_BYTES = 64 << 20


def pa_decode_split_noalloc(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                            value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                            scale: float, max_context_len: int, partition_size: int,
                            lse_out: torch.Tensor | None = None, stream=None) -> None:
    """pa_decode_split with the library's own per-GPU device array as workspace
    (no allocation; at most PA_DECODE_SPLIT_NOALLOC_MAX_BYTES of workspace)."""
    p, (S, Hq, Hkv, d, NB, bs, MB) = _decode_common(out, query, key_cache, value_cache, block_tables,
                                                   context_lens, lse_out)
    lib = load_library()
    _invoke(lib.pa_decode_split_noalloc, "pa_decode_split_noalloc", p["out"], p["query"], p["kc"], p["vc"], p["bt"],
            MB, p["cl"], S, Hq, Hkv, d, NB, bs, float(scale), _dtype_code(query), int(max_context_len),
            int(partition_size), p["lse"], _stream(stream))


def workspace_views(workspace: torch.Tensor, num_seqs: int, num_heads: int, head_size: int,
                    max_context_len: int, partition_size: int):
    """Views into a pa_decode_split workspace after a call.

    Returns (o_parts [S, H, slots, d] float32, lse_parts [S, H, slots] float32,
    total_blocks, num_ranges, block_prefix [S + 1] int32): the partials and the
    layout of the pieces the call used (see include/pa.h).
    """
    slots = -(-max_context_len // partition_size) + 1
    rows = num_seqs * num_heads * slots
    a256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    lse_off = a256(rows * head_size * 4)
    hdr_off = lse_off + a256(rows * 4)
    f = workspace.view(torch.uint8)
    o_parts = f[:rows * head_size * 4].view(torch.float32).view(num_seqs, num_heads, slots, head_size)
    lse_parts = f[lse_off:lse_off + rows * 4].view(torch.float32).view(num_seqs, num_heads, slots)
    hdr = f[hdr_off:hdr_off + 16].view(torch.int64).cpu()
    prefix = f[hdr_off + 16:hdr_off + 16 + 4 * (num_seqs + 1)].view(torch.int32)
    return o_parts, lse_parts, int(hdr[0]), int(hdr[1]), prefix


def pa_merge_partitions(out: torch.Tensor, o_parts: torch.Tensor, lse_parts: torch.Tensor,
                        lse_out: torch.Tensor | None = None, stream=None) -> None:
    """Log-sum-exp merge of float32 partials [S, H, P, d] / [S, H, P] into ``out`` [S, H, d]."""
    if o_parts.dim() != 4 or lse_parts.shape != o_parts.shape[:3]:
        raise ValueError("o_parts must be [S, H, P, d] and lse_parts [S, H, P]")
    S, H, P, d = (int(x) for x in o_parts.shape)
    if out.shape != (S, H, d):
        raise ValueError("out must be [S, H, d]")
    lse_ptr = None
    if lse_out is not None:
        if lse_out.shape != (S, H):
            raise ValueError("lse_out must be [S, H]")
        lse_ptr = _dev(lse_out, "lse_out", torch.float32)
    lib = load_library()
    _invoke(lib.pa_merge_partitions, "pa_merge_partitions", _dev(out, "out"), lse_ptr,
            _dev(o_parts, "o_parts", torch.float32), _dev(lse_parts, "lse_parts", torch.float32), S, H, P, d,
            _dtype_code(out), _stream(stream))


# ------------------------------------------------------------------ measurement kernels (include/pa_measure.h)
def pa_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of ``src`` once (the plain streaming-read ceiling); ``sink`` is int32 [>= 1]."""
    nbytes = src.numel() * src.element_size()
    lib = load_library()
    _invoke(lib.pa_stream_read, "pa_stream_read", _dev(src, "src"), nbytes, _dev(sink, "sink", torch.int32),
            _stream(stream))


def pa_stream_kv(key_cache: torch.Tensor, value_cache: torch.Tensor, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, sink: torch.Tensor, seq_order: torch.Tensor | None = None,
                 stream=None) -> None:
    """The K/V loads of pa_decode on these tables without its arithmetic (the
    decode's access-pattern ceiling); uint8 caches are FP8."""
    NB, bs, Hkv, d = _cache_dims(key_cache, value_cache)
    kind = {torch.float32: 0, torch.bfloat16: 1, torch.uint8: 2}.get(key_cache.dtype)
    if kind is None:
        raise TypeError(f"unsupported cache dtype {key_cache.dtype}")
    if block_tables.dim() != 2 or context_lens.shape != (int(block_tables.shape[0]),):
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq] and context_lens [num_seqs]")
    S = int(block_tables.shape[0])
    order_ptr = None
    if seq_order is not None:
        if seq_order.shape != (S,):
            raise ValueError("seq_order must be [num_seqs]")
        order_ptr = _dev(seq_order, "seq_order", torch.int32, 1)
    lib = load_library()
    _invoke(lib.pa_stream_kv, "pa_stream_kv", _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            _dev(block_tables, "block_tables", torch.int32, 2), int(block_tables.shape[1]),
            _dev(context_lens, "context_lens", torch.int32, 1), S, Hkv, d, NB, bs, kind, order_ptr,
            _dev(sink, "sink", torch.int32), _stream(stream))
