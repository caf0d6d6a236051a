"""GPU parity for the FP8 (E4M3) KV cache: the quantizing scatter bit-exact
against the oracle's codes, and decode over FP8 caches against the oracle's
attention on code values times the scales."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_TOL, TOL, bits, ensure_built, f64, forced, max_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


@pytest.fixture(autouse=True, params=["tiles", "tiles4"])
def decode_kernel(request, pa):
    """Run every test here with the tile kernel's own choice of waves per
    workgroup (8 on these small grids) and with 4 forced."""
    if request.param == "tiles4":
        with forced(pa, tile_waves=4):
            yield request.param
    else:
        yield request.param


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _specials(dtype, shape, rng):
    """Rows with NaN, +-inf, overflow, tiny values, signed zeros and ordinary values."""
    x = (rng.standard_normal(shape) * 2.0 ** rng.integers(-14, 12, shape)).astype(np.float32)
    flat = x.reshape(-1)
    sp = np.array([np.nan, -np.nan, np.inf, -np.inf, 1e30, -1e30, 0.0, -0.0, 3e-8, -3e-8, 448, -448,
                   465.0, 463.9, 2.0 ** -9, 2.0 ** -10], np.float32)
    flat[: sp.size] = sp
    flat[sp.size: 2 * sp.size] = sp * np.float32(1 / 64)
    return x if dtype == "f32" else W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hkv,d", [(8, 128), (2, 64)])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (1 / 64, 1 / 8), (0.3, 3.0), (2.0 ** 20, 2.0 ** -20)])
def test_reshape_fp8_bit_exact(pa, dtype, Hkv, d, scales):
    rng = np.random.default_rng(21)
    nb, T = 40, 37
    key = _specials(dtype, (T, Hkv, d), rng)
    val = _specials(dtype, (T, Hkv, d), rng)
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[::9] = -1
    slots[5] = nb * 16 + 3
    kc = rng.integers(0, 256, (nb, 16, Hkv, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, 16, Hkv, d)).astype(np.uint8)
    gk, gv = _dev_u8(kc), _dev_u8(vc)
    pa.pa_reshape_and_cache_fp8(to_dev(key), to_dev(val), gk, gv, to_dev(slots), *scales)
    torch.cuda.synchronize()
    rk, rv = oracle.reshape_and_cache_fp8(key, val, kc, vc, slots, *scales)
    np.testing.assert_array_equal(gk.cpu().numpy(), rk)
    np.testing.assert_array_equal(gv.cpu().numpy(), rv)


SWEEP = [(d, Hq, Hkv) for d in (64, 128) for Hq, Hkv in ((8, 8), (8, 4), (8, 2), (16, 4), (16, 2), (16, 1))]


@pytest.mark.parametrize("d,Hq,Hkv", SWEEP, ids=lambda v: str(v))
def test_decode_fp8_matches_the_oracle(pa, d, Hq, Hkv):
    lens = np.array([1, 15, 16, 17, 33, 100, 257, 31, 48, 129, 0], np.int32)
    cfg = W.small_case("fp8sweep", len(lens), Hq, Hkv, d, "bf16", ("uniform", 1, 2), seed=23, num_blocks=220,
                       kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 32)
    inp = W.make_inputs(cfg, context_lens=np.maximum(lens, 1))
    inp.context_lens = lens
    out = torch.empty((len(lens), Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((len(lens), Hq), dtype=torch.float32, device="cuda")
    args = (to_dev(inp.query), _dev_u8(inp.key_cache), _dev_u8(inp.value_cache), to_dev(inp.block_tables),
            to_dev(lens), cfg.scale, cfg.k_scale, cfg.v_scale)
    pa.pa_decode_fp8(out, *args, lse_out=lse)
    out2 = torch.empty_like(out)
    pa.pa_decode_fp8(out2, *args, seq_order=to_dev(np.argsort(-lens, kind="stable").astype(np.int32)))
    torch.cuda.synchronize()
    ref, ref_lse = oracle.paged_decode_fp8(inp.query, inp.key_cache, inp.value_cache, inp.block_tables, lens,
                                           cfg.scale, cfg.k_scale, cfg.v_scale)
    z = lens == 0
    assert (f64(out)[z] == 0).all() and np.isneginf(f64(lse)[z]).all()
    assert max_err(out[~torch.from_numpy(z).cuda()], ref[~z]) <= TOL["bf16"]
    assert np.abs(f64(lse)[~z] - ref_lse[~z]).max() <= LSE_TOL["bf16"]
    np.testing.assert_array_equal(bits(out), bits(out2))


def test_fp8_step_full_size(pa):
    """The FP8 batch-256 workload: quantizing write of the 256 new tokens into
    the pool, then decode; every code written is checked, and every output
    row and log-sum-exp against the oracle."""
    cfg = W.CONFIG_BY_NAME["llama3_8b_b256_fp8"]
    inp = W.make_inputs(cfg, mode="perf")
    kc_h, vc_h = W.caches_before_write(inp)
    gk, gv = _dev_u8(kc_h), _dev_u8(vc_h)
    pa.pa_reshape_and_cache_fp8(to_dev(inp.new_key), to_dev(inp.new_value), gk, gv, to_dev(inp.slot_mapping),
                                cfg.k_scale, cfg.v_scale)
    out = torch.empty((cfg.num_seqs, cfg.num_heads, cfg.head_size), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((cfg.num_seqs, cfg.num_heads), dtype=torch.float32, device="cuda")
    pa.pa_decode_fp8(out, to_dev(inp.query), gk, gv, to_dev(inp.block_tables), to_dev(inp.context_lens),
                     cfg.scale, cfg.k_scale, cfg.v_scale, lse_out=lse)
    torch.cuda.synchronize()
    rows = cfg.num_blocks * 16
    slots = inp.slot_mapping
    flat_k = gk.view(rows, cfg.num_kv_heads, cfg.head_size)[torch.from_numpy(slots).cuda()].cpu().numpy()
    flat_v = gv.view(rows, cfg.num_kv_heads, cfg.head_size)[torch.from_numpy(slots).cuda()].cpu().numpy()
    np.testing.assert_array_equal(flat_k, oracle.quantize(inp.new_key, cfg.k_scale))
    np.testing.assert_array_equal(flat_v, oracle.quantize(inp.new_value, cfg.v_scale))
    kc_after, vc_after = gk.cpu().numpy(), gv.cpu().numpy()
    ref, ref_lse = oracle.paged_decode_fp8(inp.query, kc_after, vc_after, inp.block_tables, inp.context_lens,
                                           cfg.scale, cfg.k_scale, cfg.v_scale)
    assert max_err(out, ref) <= TOL["bf16"]
    assert max_err(lse, ref_lse) <= LSE_TOL["bf16"]


def _fp8_fused(pa, q, new_k, new_v, slots, gk, gv, bt, cl, cfg):
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_reshape_and_decode_fp8(out, q, to_dev(new_k), to_dev(new_v), to_dev(slots), gk, gv, bt, cl, cfg.scale,
                                 cfg.k_scale, cfg.v_scale, lse_out=lse)
    return out, lse


@pytest.mark.parametrize("scales", [(1 / 64, 1 / 32), (0.3 / 64, 1 / 48)], ids=["pow2", "other"])
@pytest.mark.parametrize("d,Hq,Hkv", [(128, 32, 8), (64, 8, 2), (128, 16, 1)])
def test_fp8_one_launch_step_slots_and_shapes(pa, d, Hq, Hkv, scales):
    """pa_reshape_and_decode_fp8 on ragged contexts (empty, one token, block
    boundaries) with every slot case: position n-1's own slot, padding, a free
    block (the row is written, attention keeps the cached codes), past the
    pool. Rows written to free blocks carry NaN, infinities, overflow and
    subnormal values. Power-of-two scales take the reciprocal path of the
    write, others the division. Caches bit-exact against the oracle's quantizing write,
    outputs bit-identical to the two-launch step and within tolerance of the
    oracle."""
    lens = np.array([1, 15, 16, 17, 33, 100, 257, 31, 0, 48, 129, 64], np.int32)
    cfg = W.small_case("fp8fused", len(lens), Hq, Hkv, d, "bf16", ("uniform", 1, 2), seed=53, num_blocks=240,
                       kv_dtype="fp8", k_scale=scales[0], v_scale=scales[1])
    inp = W.make_inputs(cfg, context_lens=np.maximum(lens, 1))
    inp.context_lens = lens
    rows = cfg.num_blocks * 16
    free = np.setdiff1d(np.arange(cfg.num_blocks), inp.referenced_blocks)
    rng = np.random.default_rng(8)
    new_k, new_v = inp.new_key.copy(), inp.new_value.copy()
    slots = inp.slot_mapping.copy()
    kb, vb = W.caches_before_write(inp)
    keep = {1: -1, 3: int(free[0]) * 16 + 9, 8: int(free[1]) * 16 + 2, 10: rows, 11: 2 ** 40}
    for i, s in keep.items():
        if lens[i] > 0:
            # Position n-1 keeps the codes of its token already in the cache.
            kb.reshape(rows, Hkv, d)[inp.slot_mapping[i]] = oracle.quantize(inp.new_key[i], cfg.k_scale)
            vb.reshape(rows, Hkv, d)[inp.slot_mapping[i]] = oracle.quantize(inp.new_value[i], cfg.v_scale)
        new_k[i] = _specials("bf16", (Hkv, d), rng)
        new_v[i] = _specials("bf16", (Hkv, d), rng)
        slots[i] = s
    gk, gv = _dev_u8(kb), _dev_u8(vb)
    q, bt, cl = to_dev(inp.query), to_dev(inp.block_tables), to_dev(lens)
    out, lse = _fp8_fused(pa, q, new_k, new_v, slots, gk, gv, bt, cl, cfg)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.reshape_and_cache_fp8(new_k, new_v, kb, vb, slots, cfg.k_scale, cfg.v_scale)
    np.testing.assert_array_equal(gk.cpu().numpy(), ref_k)
    np.testing.assert_array_equal(gv.cpu().numpy(), ref_v)
    # Two launches on the same inputs: identical bits.
    gk2, gv2 = _dev_u8(kb), _dev_u8(vb)
    pa.pa_reshape_and_cache_fp8(to_dev(new_k), to_dev(new_v), gk2, gv2, to_dev(slots), cfg.k_scale, cfg.v_scale)
    out2 = torch.empty_like(q)
    lse2 = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    pa.pa_decode_fp8(out2, q, gk2, gv2, bt, cl, cfg.scale, cfg.k_scale, cfg.v_scale, lse_out=lse2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(out2))
    np.testing.assert_array_equal(bits(lse), bits(lse2))
    ref, ref_lse = oracle.paged_decode_fp8(inp.query, ref_k, ref_v, inp.block_tables, lens, cfg.scale, cfg.k_scale,
                                           cfg.v_scale)
    z = lens == 0
    o, l = f64(out), f64(lse)
    assert (o[z] == 0).all() and np.isneginf(l[z]).all()
    assert np.abs(o[~z] - ref[~z]).max() <= TOL["bf16"]
    assert np.abs(l[~z] - ref_lse[~z]).max() <= LSE_TOL["bf16"]


def test_fp8_one_launch_step_full_size(pa):
    """The FP8 batch-256 workload as one launch: the written codes bit-exact,
    every output row and log-sum-exp against the oracle."""
    cfg = W.CONFIG_BY_NAME["llama3_8b_b256_fp8"]
    inp = W.make_inputs(cfg, mode="perf")
    kc_h, vc_h = W.caches_before_write(inp)
    gk, gv = _dev_u8(kc_h), _dev_u8(vc_h)
    q = to_dev(inp.query)
    out, lse = _fp8_fused(pa, q, inp.new_key, inp.new_value, inp.slot_mapping, gk, gv, to_dev(inp.block_tables),
                          to_dev(inp.context_lens), cfg)
    torch.cuda.synchronize()
    rows = cfg.num_blocks * 16
    sl = torch.from_numpy(inp.slot_mapping).cuda()
    np.testing.assert_array_equal(gk.view(rows, cfg.num_kv_heads, cfg.head_size)[sl].cpu().numpy(),
                                  oracle.quantize(inp.new_key, cfg.k_scale))
    np.testing.assert_array_equal(gv.view(rows, cfg.num_kv_heads, cfg.head_size)[sl].cpu().numpy(),
                                  oracle.quantize(inp.new_value, cfg.v_scale))
    ref, ref_lse = oracle.paged_decode_fp8(inp.query, gk.cpu().numpy(), gv.cpu().numpy(), inp.block_tables,
                                           inp.context_lens, cfg.scale, cfg.k_scale, cfg.v_scale)
    assert max_err(out, ref) <= TOL["bf16"]
    assert max_err(lse, ref_lse) <= LSE_TOL["bf16"]
