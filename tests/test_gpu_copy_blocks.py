"""GPU parity for pa_copy_blocks (bit-exact against the oracle), alone and as
the GPU half of copy-on-write with the native block pool."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, Dev, bits, ensure_built, max_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


def _pairs(rng, nb, n, junk=0):
    ids = rng.permutation(nb)
    src, dst = ids[:n], ids[n:2 * n]
    pairs = np.stack([src, dst], 1).astype(np.int64)
    if junk:
        bad = np.stack([rng.integers(nb, 2 * nb, junk), rng.integers(0, nb, junk)], 1)
        bad[::2] = bad[::2, ::-1]
        bad[::3, 0] = -1
        pairs = np.concatenate([pairs, bad]).astype(np.int64)
        pairs = pairs[rng.permutation(len(pairs))]
    return pairs


@pytest.mark.parametrize("dtype,Hkv,d", [("bf16", 8, 128), ("f32", 2, 64), ("bf16", 1, 64), ("bf16", 16, 128), ("f32", 8, 128)])
def test_copy_blocks_bit_exact(pa, dtype, Hkv, d):
    rng = np.random.default_rng(11)
    nb = 300
    cfg = W.small_case("copy", 2, Hkv, Hkv, d, dtype, ("uniform", 1, 2), seed=11, num_blocks=nb)
    inp = W.make_inputs(cfg)
    kc_h, vc_h = inp.key_cache, inp.value_cache
    # make every block distinct (the generator fills only referenced blocks)
    kc_h = np.ascontiguousarray(rng.integers(0, 2**15, kc_h.shape).astype(kc_h.dtype))
    vc_h = np.ascontiguousarray(rng.integers(0, 2**15, vc_h.shape).astype(vc_h.dtype))
    pairs = _pairs(rng, nb, 120, junk=9)
    kc, vc = to_dev(kc_h), to_dev(vc_h)
    pa.pa_copy_blocks(kc, vc, to_dev(pairs))
    pa.pa_copy_blocks(kc, vc, to_dev(np.zeros((0, 2), np.int64)))
    torch.cuda.synchronize()
    rk, rv = oracle.copy_blocks(kc_h, vc_h, pairs)
    host_bits = lambda a: a.view(np.uint32) if a.dtype == np.float32 else a  # noqa: E731
    np.testing.assert_array_equal(bits(kc), host_bits(rk))
    np.testing.assert_array_equal(bits(vc), host_bits(rv))


def test_copy_on_write_end_to_end(pa):
    """Two sequences share a 40-token prefix through the native pool; the
    second gets a private copy of the partly filled block, writes its new token
    there, and both decode to the oracle's answers."""
    from paged_kv_cache_150_amd.pool import BlockPool
    rng = np.random.default_rng(12)
    cfg = W.small_case("cow", 2, 8, 2, 128, "bf16", ("uniform", 1, 2), seed=12, num_blocks=16)
    inp = W.make_inputs(cfg)
    pool = BlockPool(16, 16, free_order=rng.permutation(16))
    a = pool.allocate(40)
    b = list(a)
    pool.share(b)
    cpy = pool.make_writable(b, 2)
    assert cpy is not None
    kc_h = np.ascontiguousarray(W.f32_to_bf16_bits(rng.standard_normal(inp.key_cache.shape).astype(np.float32)))
    vc_h = np.ascontiguousarray(W.f32_to_bf16_bits(rng.standard_normal(inp.value_cache.shape).astype(np.float32)))
    kc, vc = to_dev(kc_h), to_dev(vc_h)
    pa.pa_copy_blocks(kc, vc, to_dev(np.array([cpy], np.int64)))
    newk = W.f32_to_bf16_bits(rng.standard_normal((1, 2, 128)).astype(np.float32))
    newv = W.f32_to_bf16_bits(rng.standard_normal((1, 2, 128)).astype(np.float32))
    slot = np.array([b[2] * 16 + 40 % 16], np.int64)
    pa.pa_reshape_and_cache(to_dev(newk), to_dev(newv), kc, vc, to_dev(slot))
    tables = np.array([a, b], np.int32)
    lens = np.array([40, 41], np.int32)
    inp.key_cache, inp.value_cache = bits(kc), bits(vc)
    inp.block_tables, inp.context_lens = tables, lens
    d = Dev(inp)
    out, _ = d.decode(pa)
    torch.cuda.synchronize()
    k1, v1 = oracle.copy_blocks(kc_h, vc_h, [cpy])
    k2, v2 = oracle.reshape_and_cache(newk, newv, k1, v1, slot)
    np.testing.assert_array_equal(bits(kc), k2)
    ref, _ = oracle.paged_decode(inp.query, k2, v2, tables, lens, cfg.scale, "bf16")
    assert max_err(out, ref) <= TOL["bf16"]
    # the reader's block is untouched by the writer's token
    np.testing.assert_array_equal(k2[a[2]], kc_h[a[2]])


def test_copy_blocks_full_pool_sampled(pa):
    """Pool of the batch-256 workload's shape, 4,096 pairs: checked on a sample."""
    rng = np.random.default_rng(13)
    nb, shape = 32768, (32768, 16, 8, 128)
    kc = torch.randint(-2**15, 2**15, shape, dtype=torch.int16, device="cuda")
    vc = torch.randint(-2**15, 2**15, shape, dtype=torch.int16, device="cuda")
    pairs = _pairs(rng, nb, 4096)
    before_k = kc[torch.from_numpy(pairs[:64, 0]).cuda()].clone()
    before_v = vc[torch.from_numpy(pairs[:64, 0]).cuda()].clone()
    untouched = torch.from_numpy(np.setdiff1d(np.arange(nb), pairs[:, 1])[:64]).cuda()
    keep = kc[untouched].clone()
    pa.pa_copy_blocks(kc.view(torch.bfloat16), vc.view(torch.bfloat16), to_dev(pairs))
    torch.cuda.synchronize()
    dst = torch.from_numpy(pairs[:64, 1]).cuda()
    assert torch.equal(kc[dst], before_k) and torch.equal(vc[dst], before_v)
    assert torch.equal(kc[untouched], keep)
