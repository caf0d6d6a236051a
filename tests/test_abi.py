"""The C ABI without a GPU: libpa.so loads, exports every symbol include/*.h
declares, and rejects bad arguments on the host before any GPU work is queued."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def lib():
    from gpu_helpers import ensure_built
    pa = ensure_built()
    return pa.load_library()


def declared_functions(header=None):
    names = set()
    for h in ([header] if header else HEADERS):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_headers_declare_the_boundary():
    inc = os.path.join(ROOT, "include")
    assert declared_functions(os.path.join(inc, "pa.h")) == sorted([
        "pa_reshape_and_cache", "pa_reshape_and_cache_fp8", "pa_copy_blocks", "pa_decode", "pa_decode_fp8",
        "pa_reshape_and_decode", "pa_reshape_and_decode_fp8", "pa_multi_query", "pa_multi_query_fp8", "pa_multi_query_split_workspace_bytes",
        "pa_multi_query_split", "pa_multi_query_split_partition_size", "pa_decode_prefix_workspace_bytes",
        "pa_decode_prefix",
        "pa_decode_split_workspace_bytes", "pa_decode_split", "pa_merge_partitions", "pa_status_string",
        "pa_decode_split_part_tokens", "pa_set_option", "pa_get_option", "pa_decode_split_noalloc"])
    assert declared_functions(os.path.join(inc, "pa_measure.h")) == ["pa_stream_kv", "pa_stream_read"]
    assert declared_functions(os.path.join(inc, "pa_pool.h")) == sorted([
        "pa_pool_create", "pa_pool_destroy", "pa_pool_num_free", "pa_pool_ref_count", "pa_pool_blocks_for",
        "pa_pool_allocate", "pa_pool_append_slot", "pa_pool_share", "pa_pool_release",
        "pa_pool_make_writable", "pa_prepare_step"])


def test_library_exports_every_declared_symbol(lib):
    import paged_kv_cache_150_amd as pa
    out = subprocess.run(["nm", "-D", "--defined-only", pa.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (pa_[a-z0-9_]+)\b", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_kernel_options(lib):
    """Options keep valid values, reject the rest unchanged, and read back."""
    valid = {0: [0, 4, 8], 1: [0, 16, 32], 2: [0, 1, 2], 3: [0, 1, 7], 4: [0, 1, 2, 4]}
    invalid = {0: [2, 16, -1], 1: [8, 64], 2: [3, -1], 3: [-1], 4: [3, 8]}
    for opt, vals in valid.items():
        for v in vals:
            assert lib.pa_set_option(opt, v) == 0 and lib.pa_get_option(opt) == v
        for v in invalid[opt]:
            assert lib.pa_set_option(opt, v) == 1 and lib.pa_get_option(opt) == vals[-1]
        assert lib.pa_set_option(opt, 0) == 0
    assert lib.pa_set_option(5, 0) == 1 and lib.pa_set_option(-1, 0) == 1
    assert lib.pa_get_option(5) == -1 and lib.pa_get_option(-1) == -1


def test_status_strings(lib):
    for code in range(6):
        assert lib.pa_status_string(code) != b"unknown status"
    assert lib.pa_status_string(99) == b"unknown status"


def test_workspace_size(lib):
    f = lib.pa_decode_split_workspace_bytes
    a = lambda n: (n + 255) // 256 * 256  # noqa: E731
    # 8 seqs x 32 heads x (ceil(32768/512) + 1) slots: o_p, lse_p, header, each 256-aligned.
    rows = 8 * 32 * 65
    assert f(8, 32, 128, 32768, 512) == a(rows * 128 * 4) + a(rows * 4) + a(16 + 9 * 4)
    rows = 4 * 4 * 5
    assert f(4, 4, 64, 100, 32) == a(rows * 64 * 4) + a(rows * 4) + a(16 + 5 * 4)
    assert f(1, 1, 64, 0, 16) > 0          # at least one partition
    assert f(1, 1, 64, 10, 0) == 0         # invalid partition size
    assert f(-1, 1, 64, 10, 16) == 0


P = ctypes.c_void_p


def _decode(lib, **kw):
    a = dict(out=16, query=16, kc=16, vc=16, bt=16, mb=4, cl=16, S=2, Hq=8, Hkv=2, d=128, NB=10, bs=16,
             scale=0.1, dtype=1, lse=None)
    a.update(kw)
    return lib.pa_decode(a["out"], a["query"], a["kc"], a["vc"], a["bt"], a["mb"], a["cl"], a["S"], a["Hq"],
                         a["Hkv"], a["d"], a["NB"], a["bs"], a["scale"], a["dtype"], a["lse"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 1), (dict(Hq=6, Hkv=4), 1), (dict(Hq=64, Hkv=2), 2), (dict(d=96), 2),
    (dict(bs=32), 2), (dict(out=None), 1), (dict(query=8), 1), (dict(NB=0), 1), (dict(S=-1), 1),
    (dict(mb=0), 1), (dict(S=0), 0),
])
def test_decode_host_validation(lib, kw, status):
    # Pointers are fake: every case returns before the GPU is touched.
    assert _decode(lib, **kw) == status


def test_split_and_merge_host_validation(lib):
    args = [16, 16, 16, 16, 16, 4, 16, 2, 8, 2, 128, 10, 16, ctypes.c_float(0.1), 1]
    need = lib.pa_decode_split_workspace_bytes(2, 8, 128, 64, 16)
    assert lib.pa_decode_split(*args, 64, 24, 256, need, None, None) == 1      # P % 16 != 0
    assert lib.pa_decode_split(*args, 64, 16, None, need, None, None) == 1     # no workspace
    assert lib.pa_decode_split(*args, 64, 16, 272, need, None, None) == 1      # misaligned workspace
    assert lib.pa_decode_split(*args, 64, 16, 256, need - 1, None, None) == 3  # too small
    n = lib.pa_decode_split_noalloc
    assert n(*args, 64, 24, None, None) == 1                                  # P % 16 != 0
    assert n(*args, 1 << 24, 16, None, None) == 3                             # past the array's size
    assert n(*args[:7], 0, *args[8:], 64, 16, None, None) == 0                # no sequences
    assert lib.pa_merge_partitions(16, None, 16, 16, 2, 8, 0, 128, 1, None) == 1
    assert lib.pa_merge_partitions(16, None, 16, 16, 2, 8, 3, 80, 1, None) == 2


def test_measure_host_validation(lib):
    assert lib.pa_stream_read(16, 0, 16, None) == 0                      # nothing to read
    assert lib.pa_stream_read(16, 24, 16, None) == 1                     # not a multiple of 16
    assert lib.pa_stream_read(8, 32, 16, None) == 1                      # misaligned
    assert lib.pa_stream_read(16, 32, None, None) == 1                   # no sink
    f = lib.pa_stream_kv
    assert f(16, 16, 16, 4, 16, 0, 8, 128, 10, 16, 1, None, 16, None) == 0   # no sequences
    assert f(16, 16, 16, 4, 16, 2, 8, 128, 10, 16, 3, None, 16, None) == 1   # cache kind
    assert f(16, 16, 16, 4, 16, 2, 8, 96, 10, 16, 1, None, 16, None) == 2    # head size
    assert f(16, 16, 16, 4, 16, 2, 8, 128, 10, 16, 1, None, None, None) == 1  # no sink


def test_reshape_host_validation(lib):
    f = lib.pa_reshape_and_cache
    assert f(16, 16, 16, 16, 16, 0, 10, 16, 2, 128, 1, None) == 0       # nothing to do
    assert f(16, 16, 16, 16, 16, 4, 10, 8, 2, 128, 1, None) == 2        # block size
    assert f(16, 16, 16, 16, None, 4, 10, 16, 2, 128, 1, None) == 1     # null slots
    assert f(16, 8, 16, 16, 16, 4, 10, 16, 2, 128, 1, None) == 1        # misaligned
    assert f(16, 16, 16, 16, 16, 4, 10, 16, 2, 128, 3, None) == 1       # dtype


def test_binding_refuses_host_tensors():
    import torch
    import paged_kv_cache_150_amd as pa
    from gpu_helpers import ensure_built
    ensure_built()
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    kc = torch.zeros(4, 16, 2, 128, dtype=torch.bfloat16)
    bt = torch.zeros(2, 1, dtype=torch.int32)
    cl = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        pa.pa_decode(torch.empty_like(q), q, kc, kc.clone(), bt, cl, 0.1)
    with pytest.raises(ValueError):
        pa.pa_decode(torch.empty_like(q), q, kc, kc.clone(), bt[:1], cl, 0.1)


def test_copy_blocks_host_validation(lib):
    f = lib.pa_copy_blocks
    assert f(16, 16, 16, 0, 10, 16, 2, 128, 1, None) == 0        # nothing to do
    assert f(16, 16, 16, 4, 10, 8, 2, 128, 1, None) == 2         # block size
    assert f(16, 16, None, 4, 10, 16, 2, 128, 1, None) == 1      # no mapping
    assert f(16, 8, 16, 4, 10, 16, 2, 128, 1, None) == 1         # misaligned cache
    assert f(16, 16, 16, -1, 10, 16, 2, 128, 1, None) == 1       # negative count
    assert f(16, 16, 16, 4, 10, 16, 2, 96, 1, None) == 2         # head size


def test_fp8_host_validation(lib):
    f = lib.pa_reshape_and_cache_fp8
    c = ctypes.c_float
    assert f(16, 16, 16, 16, 16, 0, 10, 16, 2, 128, 1, c(1.0), c(1.0), None) == 0     # nothing to do
    assert f(16, 16, 16, 16, 16, 4, 10, 16, 2, 128, 1, c(0.0), c(1.0), None) == 1     # scale must be > 0
    assert f(16, 16, 16, 16, 16, 4, 10, 16, 2, 128, 1, c(1.0), c(float("nan")), None) == 1
    assert f(16, 16, 16, 12, 16, 4, 10, 16, 2, 128, 1, c(1.0), c(1.0), None) == 1     # cache not 8-aligned
    assert f(16, 16, 16, 16, 16, 4, 10, 16, 2, 128, 3, c(1.0), c(1.0), None) == 1     # dtype
    d = lib.pa_decode_fp8
    base = [16, 16, 16, 16, 16, 4, 16, 2, 8, 2, 128, 10, 16, c(0.1)]
    assert d(*base, c(1.0), c(1.0), 0, None, None, None) == 2                         # f32 query unsupported
    assert d(*base, c(-1.0), c(1.0), 1, None, None, None) == 1                        # negative scale


def test_multi_query_host_validation(lib):
    f = lib.pa_multi_query
    c = ctypes.c_float
    ok = [16, 16, 16, 16, 16, 4, 16, 16]            # out, query, caches, tables, max_blocks, lens, starts
    shape = [8, 2, 128, 10, 16]                      # H_q, H_kv, head_size, num_blocks, block_size
    assert f(*ok, 0, 5, *shape, c(0.1), 1, None, None) == 0              # no sequences: nothing launched
    assert f(*ok, 3, 0, *shape, c(0.1), 1, None, None) == 0              # no new tokens: nothing launched
    assert f(*ok, 3, 5, *shape, c(-0.1), 1, None, None) == 1             # scale must be > 0
    assert f(*ok, 3, 5, *shape, c(float("inf")), 1, None, None) == 1
    assert f(*ok, 3, -1, *shape, c(0.1), 1, None, None) == 1             # negative token count
    assert f(*ok[:7], None, 3, 5, *shape, c(0.1), 1, None, None) == 1    # no query_start_loc
    assert f(16, 8, *ok[2:], 3, 5, *shape, c(0.1), 1, None, None) == 1   # misaligned query
    assert f(*ok, 3, 5, 8, 2, 96, 10, 16, c(0.1), 1, None, None) == 2    # head size
    assert f(*ok, 3, 5, 8, 3, 128, 10, 16, c(0.1), 1, None, None) == 1   # H_q % H_kv
    assert f(*ok, 3, 5, 64, 2, 128, 10, 16, c(0.1), 1, None, None) == 2  # group above 16
    assert f(*ok, 3, 5, *shape, c(0.1), 2, None, None) == 1              # dtype


def test_split_cut_choice(lib):
    """pa_decode_split cuts into partitions of k * P tokens (tile kernel) when
    its 16-column tiles hold the group: always with bf16 caches; with float32
    caches when the group is above 4 or the batch has at least as many
    (sequence, kv head) pairs as resident tile workgroups, else into pieces;
    the overrides win where they apply. Host-only: with no device the CU count
    defaults to 256 (512 resident tile workgroups)."""
    f = lib.pa_decode_split_part_tokens
    PART_FACTOR, CUT = 3, 2
    BF16, F32 = 1, 0
    lib.pa_set_option(PART_FACTOR, 1)
    assert f(64, 32, 8, 2048, 512, F32) == 512            # 512 pairs: partitions
    assert f(8, 32, 8, 32768, 512, F32) == 0              # 64 pairs, group 4, float32: pieces
    assert f(8, 32, 8, 32768, 512, BF16) == 512           # ... bf16: partitions
    assert f(8, 64, 8, 32768, 512, F32) == 512            # 64 pairs, group 8: partitions
    assert f(256, 64, 2, 4096, 512, BF16) == 0            # group of 32: pieces
    lib.pa_set_option(PART_FACTOR, 3)
    assert f(64, 32, 8, 32768, 512, BF16) == 1536
    assert f(64, 32, 8, 1000, 512, BF16) == 1024          # k capped at ceil(1000 / 512)
    assert f(64, 32, 8, 300, 512, BF16) == 512
    for bad in [(8, 30, 8, 4096, 512, BF16), (8, 32, 0, 4096, 512, BF16), (8, 32, 8, -1, 512, BF16),
                (8, 32, 8, 4096, 24, BF16), (-1, 32, 8, 4096, 512, BF16), (8, 32, 8, 4096, 512, 5)]:
        assert f(*bad) == -1
    lib.pa_set_option(PART_FACTOR, 0)
    assert f(64, 32, 8, 2048, 512, BF16) == 512           # 64 * 4 * 8 / 1536 rounds down to k = 1
    assert f(256, 32, 8, 4096, 512, BF16) == 4096         # k = 10, capped at 8 partitions
    assert f(8, 32, 8, 32768, 512, BF16) == 1024          # k = 8 * 64 * 8 // 1536 = 2
    lib.pa_set_option(CUT, 2)
    assert f(64, 32, 8, 2048, 512, BF16) == 0
    lib.pa_set_option(CUT, 1)
    assert f(8, 32, 8, 32768, 512, F32) == 1024 and f(256, 64, 2, 4096, 512, BF16) == 0
    lib.pa_set_option(CUT, 0)


def test_multi_query_split_host_validation(lib):
    """Workspace sizing and the host checks of pa_multi_query_split (no GPU work)."""
    f = lib.pa_multi_query_split_workspace_bytes
    a256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    rows = 10 * 8 * 4                                 # tokens, heads, ceil(2000 / 512) slots
    assert f(10, 8, 128, 2000, 512) == a256(rows * 128 * 4) + a256(rows * 4)
    assert f(10, 8, 128, 0, 512) == a256(10 * 8 * 128 * 4) + a256(10 * 8 * 4)   # at least one slot
    assert f(10, 0, 128, 2000, 512) == 0 and f(10, 8, 128, 2000, 0) == 0 and f(-1, 8, 128, 2000, 512) == 0
    g = lib.pa_multi_query_split
    c = ctypes.c_float
    ok = [16, 16, 16, 16, 16, 4, 16, 16]            # out, query, caches, tables, max_blocks, lens, starts
    shape = [8, 2, 128, 10, 16]                      # H_q, H_kv, head_size, num_blocks, block_size
    assert g(*ok, 0, 5, *shape, c(0.1), 1, 64, 16, 256, 1 << 20, None, None) == 0    # no sequences
    assert g(*ok, 3, 5, *shape, c(0.1), 1, 64, 24, 256, 1 << 20, None, None) == 1    # P not a block multiple
    assert g(*ok, 3, 5, *shape, c(0.1), 1, 64, 16, None, 1 << 20, None, None) == 1   # no workspace
    assert g(*ok, 3, 5, *shape, c(0.1), 1, 64, 16, 264, 1 << 20, None, None) == 1    # misaligned workspace
    assert g(*ok, 3, 5, *shape, c(0.1), 1, 64, 16, 256, 16, None, None) == 3         # workspace too small
    assert g(*ok[:7], None, 3, 5, *shape, c(0.1), 1, 64, 16, 256, 1 << 20, None, None) == 1  # no query_start_loc


def test_multi_query_split_partition_choice(lib):
    """Without a GPU the library assumes 256 compute units: a step whose tiles
    give fewer workgroups than that is cut to about 6 * 256 workgroups."""
    f = lib.pa_multi_query_split_partition_size
    # 8 long sequences, 5 verify positions: 32-column tiles of 8 tokens,
    # (40 / 8 + 8) * 8 = 104 jobs -> ceil(1536 / 104) = 15 parts of 32768.
    assert f(8, 40, 32, 8, 128, 1, 32768) == 2304
    assert f(64, 320, 32, 8, 128, 1, 2048) == 0       # batch 64 fills the GPU already
    assert f(256, 1279, 32, 8, 128, 1, 4096) == 0
    assert f(8, 40, 32, 8, 128, 1, 2000) == 256       # at least 256 tokens per partition
    assert f(8, 40, 32, 8, 128, 1, 200) == 0          # one partition would hold the longest context
    assert f(0, 40, 32, 8, 128, 1, 32768) == 0 and f(8, 40, 32, 8, 96, 1, 32768) == 0
