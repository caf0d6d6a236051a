"""GPU parity for pa_reshape_and_decode (the decode step's new-token write and
attention in one launch): the caches bit-exact against the oracle's write, the
outputs against the oracle and bit-identical to the separate write + decode on
the same kernel."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_TOL, TOL, Dev, bits, ensure_built, f64, max_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


def _fused(pa, d, inp, kc, vc, slots, order=None):
    out = torch.full_like(d.q, float("nan"))
    lse = torch.full(d.q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_reshape_and_decode(out, d.q, to_dev(inp.new_key), to_dev(inp.new_value), to_dev(slots), kc, vc, d.bt, d.cl,
                             inp.cfg.scale, lse_out=lse,
                             seq_order=None if order is None else to_dev(np.asarray(order, np.int32)))
    return out, lse


@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_fused_step_on_every_workload(pa, cfg):
    inp = W.make_inputs(cfg, mode="parity")
    kb, vb = W.caches_before_write(inp)
    d = Dev(inp, key_cache=kb, value_cache=vb)
    kc, vc = to_dev(kb), to_dev(vb)
    order = np.argsort(-inp.context_lens, kind="stable")
    out, lse = _fused(pa, d, inp, kc, vc, inp.slot_mapping, order)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.reshape_and_cache(inp.new_key, inp.new_value, kb, vb, inp.slot_mapping)
    np.testing.assert_array_equal(bits(kc), ref_k.view(bits(kc[:1]).dtype))
    np.testing.assert_array_equal(bits(vc), ref_v.view(bits(vc[:1]).dtype))
    # The same kernel after a separate write: identical bits.
    pa.pa_reshape_and_cache(to_dev(inp.new_key), to_dev(inp.new_value), d.kc, d.vc, to_dev(inp.slot_mapping))
    out2, lse2 = d.decode(pa, lse=True, seq_order=order)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(out2))
    np.testing.assert_array_equal(bits(lse), bits(lse2))
    ref, ref_lse = oracle.paged_decode(inp.query, ref_k, ref_v, inp.block_tables, inp.context_lens, cfg.scale,
                                       cfg.dtype)
    assert max_err(out, ref) <= TOL[cfg.dtype]
    assert max_err(lse, ref_lse) <= LSE_TOL[cfg.dtype]


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("dtype,d_h,Hq,Hkv", [("bf16", 64, 8, 2), ("f32", 128, 16, 4), ("bf16", 128, 12, 4),
                                              ("f32", 64, 16, 16)])
def test_fused_step_shapes_padding_and_empty(pa, dtype, d_h, Hq, Hkv, waves):
    """Ragged contexts (block boundaries, one token, empty) and padding slots
    (-1: nothing written, the cache already holds the token); 4- and 8-wave
    workgroups (fp32 caches run 4)."""
    pa.pa_set_option(pa.PA_OPT_TILE_WAVES, int(waves))
    lens = np.array([1, 15, 16, 17, 33, 100, 257, 31, 0, 48], np.int32)
    cfg = W.small_case("fused", len(lens), Hq, Hkv, d_h, dtype, ("uniform", 1, 2), seed=61, num_blocks=160)
    inp = W.make_inputs(cfg, context_lens=np.maximum(lens, 1))
    inp.context_lens = lens
    slots = inp.slot_mapping.copy()
    slots[lens == 0] = -1
    kb, vb = W.caches_before_write(inp)
    # Sequences 3 and 5 keep their token in the cache and pass no slot.
    for i in (3, 5):
        s = inp.slot_mapping[i]
        kb.reshape(-1, Hkv, d_h)[s] = inp.new_key[i]
        vb.reshape(-1, Hkv, d_h)[s] = inp.new_value[i]
        slots[i] = -1
    d = Dev(inp, key_cache=kb, value_cache=vb)
    kc, vc = to_dev(kb), to_dev(vb)
    out, lse = _fused(pa, d, inp, kc, vc, slots)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.reshape_and_cache(inp.new_key, inp.new_value, kb, vb, slots)
    np.testing.assert_array_equal(bits(kc), ref_k.view(bits(kc[:1]).dtype))
    ref, ref_lse = oracle.paged_decode(inp.query, ref_k, ref_v, inp.block_tables, lens, cfg.scale, dtype)
    z = lens == 0
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    assert (o[z] == 0).all() and np.isneginf(l[z]).all()
    assert np.abs(o[~z] - ref[~z]).max() <= TOL[dtype]
    assert np.abs(l[~z] - ref_lse[~z]).max() <= LSE_TOL[dtype]


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("dtype,d_h,Hq,Hkv", [("bf16", 128, 32, 8), ("f32", 64, 8, 2)])
def test_fused_step_slots_off_position_and_out_of_pool(pa, dtype, d_h, Hq, Hkv, waves):
    """Slots that are not position n-1's own: a slot in a free block (the row is
    written, attention keeps what the cache holds at n-1), an empty context
    with a slot (written), slots at and far past the pool's end (nothing
    written). The new rows of these sequences differ from the cached ones, so a
    swap into the registers would show. Caches bit-exact against the oracle's
    write; every row against the oracle and bit-identical to the separate write
    followed by pa_decode."""
    pa.pa_set_option(pa.PA_OPT_TILE_WAVES, int(waves))
    lens = np.array([40, 17, 0, 33, 100, 16, 1, 64, 31, 2], np.int32)
    cfg = W.small_case("fused_off", len(lens), Hq, Hkv, d_h, dtype, ("uniform", 1, 2), seed=67, num_blocks=96)
    inp = W.make_inputs(cfg, context_lens=np.maximum(lens, 1))
    inp.context_lens = lens
    rows = cfg.num_blocks * cfg.block_size
    free = np.setdiff1d(np.arange(cfg.num_blocks), inp.referenced_blocks)
    assert free.size >= 2
    rng = np.random.default_rng(5)
    new_k, new_v = inp.new_key.copy(), inp.new_value.copy()
    slots = inp.slot_mapping.copy()
    kb, vb = W.caches_before_write(inp)
    flat_kb, flat_vb = kb.reshape(rows, Hkv, d_h), vb.reshape(rows, Hkv, d_h)
    off = {0: int(free[0]) * 16 + 5,      # a free block
           2: int(free[1]) * 16,          # empty context, slot in a free block
           5: rows,                       # first slot past the pool
           6: 2 ** 62,                    # far past it
           8: -7}                         # padding
    for i, s in off.items():
        if lens[i] > 0:
            # Position n-1 keeps its token in the cache; the write carries other values.
            flat_kb[inp.slot_mapping[i]] = inp.new_key[i]
            flat_vb[inp.slot_mapping[i]] = inp.new_value[i]
        fresh = W.make_inputs(W.small_case("fresh", 1, Hkv, Hkv, d_h, dtype, ("uniform", 1, 1), seed=100 + i,
                                           num_blocks=1))
        new_k[i], new_v[i] = fresh.new_key[0], fresh.new_value[0]
        slots[i] = s
    assert not np.array_equal(new_k[0], inp.new_key[0])
    d = Dev(inp, key_cache=kb, value_cache=vb)
    kc, vc = to_dev(kb), to_dev(vb)
    out = torch.full_like(d.q, float("nan"))
    lse = torch.full(d.q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_reshape_and_decode(out, d.q, to_dev(new_k), to_dev(new_v), to_dev(slots), kc, vc, d.bt, d.cl, cfg.scale,
                             lse_out=lse)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.reshape_and_cache(new_k, new_v, kb, vb, slots)
    np.testing.assert_array_equal(bits(kc), ref_k.view(bits(kc[:1]).dtype))
    np.testing.assert_array_equal(bits(vc), ref_v.view(bits(vc[:1]).dtype))
    # The separate write then pa_decode: identical bits.
    pa.pa_reshape_and_cache(to_dev(new_k), to_dev(new_v), d.kc, d.vc, to_dev(slots))
    out2, lse2 = d.decode(pa, lse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(out2))
    np.testing.assert_array_equal(bits(lse), bits(lse2))
    ref, ref_lse = oracle.paged_decode(inp.query, ref_k, ref_v, inp.block_tables, lens, cfg.scale, dtype)
    z = lens == 0
    o, l = f64(out), f64(lse)
    assert (o[z] == 0).all() and np.isneginf(l[z]).all()
    assert np.abs(o[~z] - ref[~z]).max() <= TOL[dtype]
    assert np.abs(l[~z] - ref_lse[~z]).max() <= LSE_TOL[dtype]
