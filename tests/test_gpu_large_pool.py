"""GPU parity on caches larger than 4 GiB each: every byte offset the kernels
form for the blocks used here lies past 2^32 (or just below it), so 32-bit
address arithmetic anywhere in reshape_and_cache, the decode kernels, the
split path, the one-launch step or the block copy would show.

The pool is filled with NaN on the device; the referenced blocks are those of
a small workload drawn over a compact pool, placed at the top of the large
one (compact block b -> block base + b), so the host and the oracle only ever
hold the compact pool."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_TOL, TOL, bits, ensure_built, f64, forced, max_err, to_dev

pytestmark = pytest.mark.gpu

BLOCK_BYTES = 16 * 8 * 128 * 2          # one bf16 block, 8 kv heads of 128
BASE = (1 << 32) // BLOCK_BYTES - 8     # compact block 8 starts exactly at 4 GiB


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


@pytest.fixture(scope="module")
def case():
    lens = np.random.default_rng(71).integers(1, 900, 12).astype(np.int32)
    lens[:3] = [1, 16, 17]
    cfg = W.small_case("large_pool", len(lens), 32, 8, 128, "bf16", ("uniform", 1, 2), seed=71, num_blocks=1024,
                       partition_size=64)
    inp = W.make_inputs(cfg, context_lens=lens)
    nb = BASE + cfg.num_blocks
    assert nb * BLOCK_BYTES > (1 << 32) and inp.referenced_blocks.min() + BASE < (1 << 32) // BLOCK_BYTES
    return cfg, inp, nb


def _big_pool(nb, compact_k, compact_v):
    kc = torch.full((nb, 16, 8, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kc[BASE:] = to_dev(compact_k)
    vc[BASE:] = to_dev(compact_v)
    return kc, vc


def _check_pool(kc, vc, ref_k, ref_v):
    """The compact region bit-exact; everything below it still NaN."""
    np.testing.assert_array_equal(bits(kc[BASE:]), ref_k)
    np.testing.assert_array_equal(bits(vc[BASE:]), ref_v)
    assert bool(torch.isnan(kc[:BASE]).all()) and bool(torch.isnan(vc[:BASE]).all())


def test_large_pool_reshape_decode_split(pa, case):
    cfg, inp, nb = case
    print(f"[large_pool] {nb} blocks, {nb * BLOCK_BYTES / 2**30:.2f} GiB per cache", flush=True)
    kb, vb = W.caches_before_write(inp)
    kc, vc = _big_pool(nb, kb, vb)
    bt = to_dev(np.where(inp.block_tables >= 0, inp.block_tables + BASE, -1).astype(np.int32))
    cl, q = to_dev(inp.context_lens), to_dev(inp.query)
    slots = to_dev(inp.slot_mapping + BASE * 16)
    pa.pa_reshape_and_cache(to_dev(inp.new_key), to_dev(inp.new_value), kc, vc, slots)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.reshape_and_cache(inp.new_key, inp.new_value, kb, vb, inp.slot_mapping)
    _check_pool(kc, vc, ref_k, ref_v)
    ref, ref_lse = oracle.paged_decode(inp.query, ref_k, ref_v, inp.block_tables, inp.context_lens, cfg.scale,
                                       "bf16")
    S, Hq, d = inp.query.shape
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    pa.pa_decode(out, q, kc, vc, bt, cl, cfg.scale, lse_out=lse)
    torch.cuda.synchronize()
    assert max_err(out, ref) <= TOL["bf16"] and max_err(lse, ref_lse) <= LSE_TOL["bf16"]
    mcl = inp.max_context_len
    ws = torch.empty(pa.pa_decode_split_workspace_bytes(S, Hq, d, mcl, 64), dtype=torch.uint8, device="cuda")
    for cut in (1, 2):
        with forced(pa, split_cut=cut):
            out_s = torch.full_like(q, float("nan"))
            lse_s = torch.full((S, Hq), float("nan"), dtype=torch.float32, device="cuda")
            pa.pa_decode_split(out_s, q, kc, vc, bt, cl, cfg.scale, mcl, 64, ws, lse_out=lse_s)
            torch.cuda.synchronize()
        assert max_err(out_s, ref) <= TOL["bf16"] and max_err(lse_s, ref_lse) <= LSE_TOL["bf16"], cut
    # Multi-query over the same pool: the last three positions of every
    # sequence with at least three tokens, one token for the others.
    ql = np.minimum(inp.context_lens, 3).astype(np.int32)
    loc = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    qm = np.concatenate([np.repeat(inp.query[i:i + 1], ql[i], 0) for i in range(S)])
    out_m = torch.empty((int(loc[-1]), Hq, d), dtype=torch.bfloat16, device="cuda")
    pa.pa_multi_query(out_m, to_dev(qm), kc, vc, bt, cl, to_dev(loc), cfg.scale)
    torch.cuda.synchronize()
    ref_m, _ = oracle.paged_multi_query(qm, ref_k, ref_v, inp.block_tables, inp.context_lens, loc, cfg.scale,
                                        "bf16")
    assert max_err(out_m, ref_m) <= TOL["bf16"]


def test_large_pool_fused_step_and_block_copy(pa, case):
    cfg, inp, nb = case
    kb, vb = W.caches_before_write(inp)
    kc, vc = _big_pool(nb, kb, vb)
    bt = to_dev(np.where(inp.block_tables >= 0, inp.block_tables + BASE, -1).astype(np.int32))
    cl, q = to_dev(inp.context_lens), to_dev(inp.query)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    pa.pa_reshape_and_decode(out, q, to_dev(inp.new_key), to_dev(inp.new_value),
                             to_dev(inp.slot_mapping + BASE * 16), kc, vc, bt, cl, cfg.scale, lse_out=lse)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.reshape_and_cache(inp.new_key, inp.new_value, kb, vb, inp.slot_mapping)
    _check_pool(kc, vc, ref_k, ref_v)
    ref, ref_lse = oracle.paged_decode(inp.query, ref_k, ref_v, inp.block_tables, inp.context_lens, cfg.scale,
                                       "bf16")
    assert max_err(out, ref) <= TOL["bf16"] and max_err(lse, ref_lse) <= LSE_TOL["bf16"]
    # Copy-on-write copies from referenced blocks into free ones, the top
    # block of the pool included.
    free = np.setdiff1d(np.arange(cfg.num_blocks), inp.referenced_blocks)
    rng = np.random.default_rng(3)
    src = rng.choice(inp.referenced_blocks, 40, replace=False)
    dst = np.concatenate([[cfg.num_blocks - 1] if cfg.num_blocks - 1 in free else [],
                          rng.choice(free[free != cfg.num_blocks - 1], 40, replace=False)])[:40]
    pairs = np.stack([src, dst], 1).astype(np.int64)
    pa.pa_copy_blocks(kc, vc, to_dev(pairs + BASE))
    torch.cuda.synchronize()
    ck, cv = oracle.copy_blocks(ref_k, ref_v, pairs)
    _check_pool(kc, vc, ck, cv)
