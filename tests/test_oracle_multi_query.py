"""Pins for the oracle's multi-query paged attention (CPU only): an explicit
causal mask over the whole gathered context computed from scratch, the
decode of the truncated sequence for every token, one-token queries equal to
decode, and invariance under moving the physical blocks."""
import numpy as np

import oracle
import workloads as W


def _case(seed=3, dtype="bf16", Hq=8, Hkv=2, d=64):
    rng = np.random.default_rng(seed)
    cfg = W.small_case("mq", 4, Hq, Hkv, d, dtype, ("uniform", 20, 90), seed=seed, num_blocks=40)
    inp = W.make_inputs(cfg)
    qlens = np.array([1, 5, 17, 3])
    qlens = np.minimum(qlens, inp.context_lens)
    loc = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    query = W._values(rng, (int(loc[-1]), Hq, d), dtype)
    return cfg, inp, query, loc


def test_matches_an_explicit_causal_mask():
    cfg, inp, query, loc = _case()
    out, lse = oracle.paged_multi_query(query, inp.key_cache, inp.value_cache, inp.block_tables,
                                        inp.context_lens, loc, cfg.scale, "bf16")
    g = cfg.num_heads // cfg.num_kv_heads
    qf = oracle.decode_values(query, "bf16")
    for i in range(cfg.num_seqs):
        n = int(inp.context_lens[i])
        K = np.stack([oracle.decode_values(inp.key_cache[inp.block_tables[i, p // 16], p % 16], "bf16")
                      for p in range(n)])
        V = np.stack([oracle.decode_values(inp.value_cache[inp.block_tables[i, p // 16], p % 16], "bf16")
                      for p in range(n)])
        rows = np.arange(loc[i], loc[i + 1])
        qpos = n - len(rows) + np.arange(len(rows))
        allowed = np.arange(n)[None, :] <= qpos[:, None]          # [q, n]
        for h in range(cfg.num_heads):
            s = cfg.scale * qf[rows, h] @ K[:, h // g].T            # [q, n]
            s = np.where(allowed, s, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            ref = (w / w.sum(axis=1, keepdims=True)) @ V[:, h // g]
            assert np.allclose(out[rows, h], ref, atol=1e-12)
            assert np.allclose(lse[rows, h], s.max(axis=1) + np.log(w.sum(axis=1)), atol=1e-12)


def test_each_token_is_the_decode_of_its_prefix():
    cfg, inp, query, loc = _case(seed=4)
    out, lse = oracle.paged_multi_query(query, inp.key_cache, inp.value_cache, inp.block_tables,
                                        inp.context_lens, loc, cfg.scale, "bf16")
    for i in range(cfg.num_seqs):
        n = int(inp.context_lens[i])
        q = int(loc[i + 1] - loc[i])
        for j in range(q):
            t = loc[i] + j
            o1, l1 = oracle.paged_decode(query[t:t + 1], inp.key_cache, inp.value_cache,
                                         inp.block_tables[i:i + 1], np.array([n - q + j + 1]), cfg.scale, "bf16")
            assert np.allclose(out[t], o1[0], atol=1e-13) and np.allclose(lse[t], l1[0], atol=1e-13)


def test_one_token_queries_are_decode():
    cfg, inp, _, _ = _case(seed=5)
    loc = np.arange(cfg.num_seqs + 1, dtype=np.int32)
    out, lse = oracle.paged_multi_query(inp.query[:, :, :], inp.key_cache, inp.value_cache, inp.block_tables,
                                        inp.context_lens, loc, cfg.scale, "bf16")
    ref, ref_lse = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                       inp.context_lens, cfg.scale, "bf16")
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


def test_block_placement_does_not_matter():
    cfg, inp, query, loc = _case(seed=6, dtype="f32")
    out, lse = oracle.paged_multi_query(query, inp.key_cache, inp.value_cache, inp.block_tables,
                                        inp.context_lens, loc, cfg.scale, "f32")
    perm = np.random.default_rng(1).permutation(cfg.num_blocks)
    inv = np.argsort(perm)
    kc, vc = inp.key_cache[perm], inp.value_cache[perm]
    bt = np.where(inp.block_tables >= 0, inv[np.maximum(inp.block_tables, 0)], -1)
    out2, lse2 = oracle.paged_multi_query(query, kc, vc, bt, inp.context_lens, loc, cfg.scale, "f32")
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_too_many_new_tokens_see_nothing():
    cfg, inp, query, _ = _case(seed=7)
    n = inp.context_lens.copy()
    n[0] = 2
    loc = np.array([0, 4, 5, 6, 7], np.int32)
    out, lse = oracle.paged_multi_query(query[:7], inp.key_cache, inp.value_cache, inp.block_tables, n, loc,
                                        cfg.scale, "bf16")
    assert (out[:2] == 0).all() and np.isneginf(lse[:2]).all() and np.isfinite(lse[2:4]).all()
