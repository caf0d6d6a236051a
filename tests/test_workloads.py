"""Host-side checks of the seeded input generator (no GPU, no oracle arithmetic)."""
import numpy as np
import pytest
import torch

import workloads as W


def test_five_configs_shapes():
    c = W.CONFIG_BY_NAME
    assert [x.name for x in W.CONFIGS] == ["tiny_f32", "llama3_8b_b64", "llama3_8b_b256",
                                          "long_split", "prefix_70b"]
    assert c["tiny_f32"].dtype == "f32" and c["tiny_f32"].scale == 1 / 8
    for x in W.CONFIGS:
        if x.name == "tiny_f32":
            continue
        assert x.dtype == "bf16" and x.head_size == 128 and x.num_kv_heads == 8
    assert c["prefix_70b"].group == 8 and c["llama3_8b_b256"].group == 4
    assert [x.seed for x in W.CONFIGS] == [0, 1, 2, 3, 4]


@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_context_length_ranges_and_pool_fit(cfg):
    n = W.draw_context_lens(cfg)
    assert n.shape == (cfg.num_seqs,) and n.dtype == np.int32
    kind = cfg.ctx[0]
    if kind == "uniform":
        assert n.min() >= cfg.ctx[1] and n.max() <= cfg.ctx[2]
    elif kind == "normal":
        assert n.min() >= cfg.ctx[3] and n.max() <= cfg.ctx[4]
        assert abs(n.mean() - cfg.ctx[1]) < 4 * cfg.ctx[2] / np.sqrt(cfg.num_seqs)
    else:
        assert n.min() >= cfg.ctx[1] + cfg.ctx[2] and n.max() <= cfg.ctx[1] + cfg.ctx[3]
    nblk = (n + 15) // 16
    shared = cfg.ctx[1] // 16 if kind == "prefix" else 0
    assert shared + (nblk - shared).sum() <= cfg.num_blocks


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0, 3e38], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_generator_deterministic_and_layout():
    cfg = W.CONFIG_BY_NAME["tiny_f32"]
    a = W.make_inputs(cfg)
    b = W.make_inputs(cfg)
    for k in ["context_lens", "block_tables", "query", "key_cache", "value_cache", "slot_mapping"]:
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    assert a.key_cache.shape == (64, 16, 2, 64) and a.query.shape == (4, 4, 64)
    S = cfg.num_seqs
    used = []
    for i in range(S):
        n = int(a.context_lens[i])
        nb = (n + 15) // 16
        row = a.block_tables[i]
        assert (row[:nb] >= 0).all() and (row[nb:] == -1).all()
        used.extend(row[:nb].tolist())
        # New token = position n-1, through the table.
        assert a.slot_mapping[i] == row[(n - 1) // 16] * 16 + (n - 1) % 16
        np.testing.assert_array_equal(a.new_key[i], a.key_cache.reshape(-1, 2, 64)[a.slot_mapping[i]])
        # Tail slots of the last block are poisoned, valid ones finite.
        last = row[nb - 1]
        k = n - (nb - 1) * 16
        assert np.isfinite(a.key_cache[last, :k]).all()
        assert np.isnan(a.key_cache[last, k:]).all() and np.isnan(a.value_cache[last, k:]).all()
    assert len(used) == len(set(used))  # no sharing in this config
    free = np.setdiff1d(np.arange(64), used)
    assert np.isnan(a.key_cache[free]).all()
    perf = W.make_inputs(cfg, mode="perf")
    np.testing.assert_array_equal(perf.block_tables, a.block_tables)
    assert (perf.key_cache[free] == 0).all()


def test_prefix_sharing_layout_small():
    cfg = W.PagedConfig(name="p", num_seqs=6, num_heads=8, num_kv_heads=2, head_size=64,
                        block_size=16, num_blocks=128, dtype="bf16", ctx=("prefix", 64, 5, 40),
                        seed=3)
    a = W.make_inputs(cfg)
    assert a.shared_prefix_blocks == 4
    assert (a.block_tables[:, :4] == a.block_tables[0, :4]).all()
    private = [set(a.block_tables[i, 4:(a.context_lens[i] + 15) // 16].tolist()) for i in range(6)]
    for i in range(6):
        for j in range(i + 1, 6):
            assert not (private[i] & private[j])
    assert W.unique_kv_bytes(a) < W.algorithmic_kv_bytes(cfg, a.context_lens)


def test_algorithmic_bytes():
    cfg = W.CONFIG_BY_NAME["llama3_8b_b256"]
    n = np.array([1000, 10], np.int32)
    assert W.algorithmic_kv_bytes(cfg, n) == 1010 * 4096


@pytest.mark.parametrize("name", [c.name for c in W.MQ_CONFIGS])
def test_multi_query_lengths(name):
    """Each multi-query workload's lengths: every sequence has at least one new
    token and at least as many stored keys, the contexts fit the block tables
    and the pool, and the step has the new-token count its description gives."""
    cfg = W.MQ_CONFIG_BY_NAME[name]
    base = cfg.base
    n, q = W.multi_lengths(cfg)
    assert n.shape == q.shape == (base.num_seqs,)
    assert (q >= 1).all() and (n >= q).all()
    bs = base.block_size
    assert int(np.ceil(n / bs).sum()) <= base.num_blocks
    kind = cfg.new_tokens[0]
    if kind == "fixed":
        assert (q == cfg.new_tokens[1]).all()
    else:
        _, m, c, ctx = cfg.new_tokens
        assert (q[:m] == c).all() and (n[:m] == ctx).all() and (q[m:] == 1).all()
    np.testing.assert_array_equal(W.multi_lengths(cfg)[0], n)   # deterministic


def test_contiguous_placement_keeps_every_context():
    """Laying the blocks end to end renumbers them only: the oracle's decode is
    bit-identical, the new ids are 0..k-1, and every slot lands in its block."""
    import oracle
    for name in ("tiny_f32", "prefix_70b"):
        cfg = W.CONFIG_BY_NAME[name]
        inp = W.make_inputs(cfg)
        ids, tables, slots = W.contiguous_placement(inp)
        assert sorted(set(tables[tables >= 0].ravel().tolist())) == list(range(ids.size))
        ok = inp.slot_mapping >= 0
        np.testing.assert_array_equal(ids[slots[ok] // 16], inp.slot_mapping[ok] // 16)
        np.testing.assert_array_equal(slots[ok] % 16, inp.slot_mapping[ok] % 16)
        a = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables, inp.context_lens,
                                cfg.scale, cfg.dtype)[0]
        b = oracle.paged_decode(inp.query, inp.key_cache[ids], inp.value_cache[ids], tables, inp.context_lens,
                                cfg.scale, cfg.dtype)[0]
        np.testing.assert_array_equal(a, b)


def test_reorder_multi_inputs_moves_whole_sequences():
    """Reordering a multi-query step moves each sequence's table, length,
    query rows, slots and new K/V rows together: the oracle's rows of the
    reordered step are the original rows, permuted, bit for bit."""
    import oracle
    base = W.small_case("reorder", 6, 8, 2, 64, "bf16", ("uniform", 1, 2), seed=3, num_blocks=64)
    cfg = W.MultiQueryConfig("reorder", base, ("fixed", 1))
    mq = W.make_multi_inputs(cfg, context_lens=np.array([5, 40, 17, 1, 33, 9], np.int32),
                             query_lens=np.array([2, 1, 3, 1, 0, 4], np.int32))
    order = np.argsort(-mq.paged.context_lens, kind="stable")
    r = W.reorder_multi_inputs(mq, order)
    assert list(r.paged.context_lens) == sorted(mq.paged.context_lens, reverse=True)
    assert r.query_start_loc[0] == 0 and r.query_start_loc[-1] == mq.num_tokens
    rows = np.concatenate([np.arange(mq.query_start_loc[i], mq.query_start_loc[i + 1]) for i in order])
    np.testing.assert_array_equal(r.slot_mapping, mq.slot_mapping[rows])
    np.testing.assert_array_equal(r.new_key, mq.new_key[rows])
    p = mq.paged
    a, la = oracle.paged_multi_query(mq.query, p.key_cache, p.value_cache, p.block_tables, p.context_lens,
                                     mq.query_start_loc, p.cfg.scale, p.cfg.dtype)
    b, lb = oracle.paged_multi_query(r.query, p.key_cache, p.value_cache, r.paged.block_tables,
                                     r.paged.context_lens, r.query_start_loc, p.cfg.scale, p.cfg.dtype)
    np.testing.assert_array_equal(a[rows], b)
    np.testing.assert_array_equal(la[rows], lb)
