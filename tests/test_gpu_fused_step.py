"""GPU parity for pa_reshape_and_decode (the decode step's new-token write and
attention in one launch): the caches bit-exact against the oracle's write, the
outputs against the oracle and bit-identical to the separate write + decode on
the same kernel."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_TOL, TOL, Dev, bits, ensure_built, max_err, to_dev

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
def test_fused_step_on_every_workload(pa, monkeypatch, cfg):
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
    monkeypatch.setenv("PA_DECODE_KERNEL", "tiles")
    pa.pa_reshape_and_cache(to_dev(inp.new_key), to_dev(inp.new_value), d.kc, d.vc, to_dev(inp.slot_mapping))
    out2, lse2 = d.decode(pa, lse=True, seq_order=order)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(out2))
    np.testing.assert_array_equal(bits(lse), bits(lse2))
    rows = np.arange(cfg.num_seqs) if cfg.num_seqs <= 64 else np.random.default_rng(0).choice(cfg.num_seqs, 24,
                                                                                             replace=False)
    ref, ref_lse = oracle.paged_decode(inp.query[rows], ref_k, ref_v, inp.block_tables[rows],
                                       inp.context_lens[rows], cfg.scale, cfg.dtype)
    assert max_err(out[torch.from_numpy(rows).cuda()], ref) <= TOL[cfg.dtype]
    assert max_err(lse[torch.from_numpy(rows).cuda()], ref_lse) <= LSE_TOL[cfg.dtype]


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("dtype,d_h,Hq,Hkv", [("bf16", 64, 8, 2), ("f32", 128, 16, 4), ("bf16", 128, 12, 4),
                                              ("f32", 64, 16, 16)])
def test_fused_step_shapes_padding_and_empty(pa, monkeypatch, dtype, d_h, Hq, Hkv, waves):
    """Ragged contexts (block boundaries, one token, empty), padding slots
    (-1: nothing written, the cache already holds the token) and a slot past
    the pool (skipped); 4- and 8-wave workgroups (fp32 caches run 4)."""
    monkeypatch.setenv("PA_MQ_WAVES", waves)
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
