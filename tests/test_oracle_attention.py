"""Pins of the oracle's paged decode attention, LSE merge and reshape_and_cache.

The oracle is checked against things other than itself: a brute-force loop
over contiguous K/V written here, torch's scaled_dot_product_attention in fp64,
closed forms (one token, one-hot logits, uniform weights), and invariances the
pages state (placement of physical blocks does not matter; sequences may share
blocks). Each test is chosen so a plausible slip in the oracle (dropped scale,
wrong kv-head index, K/V swapped, off-by-one context length, wrong slot
formula, sign error in the merge) fails it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import f32_to_bf16_bits, bf16_bits_to_f32


# ----------------------------------------------------------------- helpers
def brute_attention(q, K, V, scale):
    """Naive per-head loop over a contiguous context (python floats)."""
    Hq, d = q.shape
    n, Hkv, _ = K.shape
    g = Hq // Hkv
    out = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    for h in range(Hq):
        kvh = h // g
        s = [scale * sum(float(q[h, e]) * float(K[t, kvh, e]) for e in range(d)) for t in range(n)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        l = sum(w)
        for e in range(d):
            out[h, e] = sum(w[t] * float(V[t, kvh, e]) for t in range(n)) / l
        lse[h] = m + math.log(l)
    return out, lse


def scatter_into_pool(Ks, Vs, num_blocks, bs, rng, poison=np.nan, share_first=0):
    """Place contiguous per-sequence K/V into a shuffled pool (independent of the oracle).

    Ks[i]: [n_i, Hkv, d]. Returns key_cache, value_cache, block_tables, context_lens.
    ``share_first`` > 0 makes every sequence reuse sequence 0's first blocks
    (their contents must then be identical across sequences).
    """
    S = len(Ks)
    Hkv, d = Ks[0].shape[1:]
    kc = np.full((num_blocks, bs, Hkv, d), poison)
    vc = np.full((num_blocks, bs, Hkv, d), poison)
    ids = list(rng.permutation(num_blocks))
    nblk = [(k.shape[0] + bs - 1) // bs for k in Ks]
    bt = np.full((S, max(max(nblk), 1)), -1, np.int32)
    for i in range(S):
        for j in range(nblk[i]):
            if j < share_first and i > 0:
                bt[i, j] = bt[0, j]
                continue
            b = ids.pop()
            bt[i, j] = b
            rows = Ks[i][j * bs:(j + 1) * bs]
            kc[b, :rows.shape[0]] = rows
            vc[b, :rows.shape[0]] = Vs[i][j * bs:(j + 1) * bs]
    return kc, vc, bt, np.array([k.shape[0] for k in Ks], np.int32)


def rand_case(rng, S, Hq, Hkv, d, lens):
    q = rng.standard_normal((S, Hq, d))
    Ks = [rng.standard_normal((n, Hkv, d)) for n in lens]
    Vs = [rng.standard_normal((n, Hkv, d)) for n in lens]
    return q, Ks, Vs


# ----------------------------------------------------------------- c-i brute force
@pytest.mark.parametrize("Hq,Hkv,d,lens,scale", [
    (4, 2, 8, [1, 5, 16, 17, 33], 0.37),
    (2, 2, 4, [3, 40], 1.0),
    (8, 1, 6, [31, 2], 0.5),
])
def test_matches_brute_force(Hq, Hkv, d, lens, scale):
    rng = np.random.default_rng(11)
    q, Ks, Vs = rand_case(rng, len(lens), Hq, Hkv, d, lens)
    kc, vc, bt, n = scatter_into_pool(Ks, Vs, 24, 16, rng)
    out, lse = _oracle_f64(q, kc, vc, bt, n, scale)
    for i in range(len(lens)):
        bo, bl = brute_attention(q[i], Ks[i], Vs[i], scale)
        np.testing.assert_allclose(out[i], bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[i], bl, rtol=0, atol=1e-12)


def _oracle_f64(q, kc, vc, bt, n, scale, bs=16):
    """The oracle's gather + attention applied to float64 pools.

    paged_decode() decodes stored bf16/f32 values first; these test pools are
    already float64, so the two building blocks it chains are called directly.
    """
    S, Hq, d = q.shape
    out = np.zeros((S, Hq, d))
    lse = np.zeros((S, Hq))
    for i in range(S):
        Kc, Vc = oracle.gather_context(kc, vc, bt[i], int(n[i]), bs)
        out[i], lse[i] = oracle.attention_contiguous(q[i], Kc, Vc, scale)
    return out, lse


def test_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(5)
    Hq, Hkv, d, n = 8, 2, 16, 45
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((n, Hkv, d))
    V = rng.standard_normal((n, Hkv, d))
    scale = 1 / math.sqrt(d)
    out, _ = oracle.attention_contiguous(q, K, V, scale)
    g = Hq // Hkv
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, dim=0)  # [Hq, n, d]
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, dim=0)
    qt = torch.from_numpy(q)[:, None, :]                                     # [Hq, 1, d]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[:, 0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def test_stored_dtypes_decode_exactly():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(1000).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    np.testing.assert_array_equal(oracle.decode_values(bits, "bf16"),
                                  bf16_bits_to_f32(bits).astype(np.float64))
    # Against torch's own bfloat16 widening.
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.decode_values(bits, "bf16"), t)
    np.testing.assert_array_equal(oracle.decode_values(x, "f32"), x.astype(np.float64))


def test_bf16_paged_decode_matches_brute_force():
    rng = np.random.default_rng(3)
    S, Hq, Hkv, d, bs, NB = 3, 4, 2, 8, 16, 16
    lens = [7, 16, 29]
    qf = rng.standard_normal((S, Hq, d)).astype(np.float32)
    q16 = f32_to_bf16_bits(qf)
    kc = np.full((NB, bs, Hkv, d), 0x7FC0, np.uint16)
    vc = kc.copy()
    bt = np.full((S, 2), -1, np.int32)
    perm = list(rng.permutation(NB))
    Ks, Vs = [], []
    for i, n in enumerate(lens):
        K16 = f32_to_bf16_bits(rng.standard_normal((n, Hkv, d)).astype(np.float32))
        V16 = f32_to_bf16_bits(rng.standard_normal((n, Hkv, d)).astype(np.float32))
        for j in range((n + bs - 1) // bs):
            b = perm.pop()
            bt[i, j] = b
            kc[b, :min(bs, n - j * bs)] = K16[j * bs:(j + 1) * bs]
            vc[b, :min(bs, n - j * bs)] = V16[j * bs:(j + 1) * bs]
        Ks.append(bf16_bits_to_f32(K16).astype(np.float64))
        Vs.append(bf16_bits_to_f32(V16).astype(np.float64))
    scale = 0.3
    out, lse = oracle.paged_decode(q16, kc, vc, bt, np.array(lens, np.int32), scale, "bf16")
    qd = bf16_bits_to_f32(q16).astype(np.float64)
    for i in range(S):
        bo, bl = brute_attention(qd[i], Ks[i], Vs[i], scale)
        np.testing.assert_allclose(out[i], bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[i], bl, rtol=0, atol=1e-12)
    assert np.isfinite(out).all()  # NaN-poisoned tails and free blocks never read


# ----------------------------------------------------------------- c-ii / c-iii invariances
def test_block_permutation_invariance_bitwise():
    rng = np.random.default_rng(7)
    q, Ks, Vs = rand_case(rng, 3, 4, 2, 8, [20, 48, 3])
    kc, vc, bt, n = scatter_into_pool(Ks, Vs, 16, 16, rng)
    out1, lse1 = _oracle_f64(q, kc, vc, bt, n, 0.4)
    pi = rng.permutation(16)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    bt2 = np.where(bt >= 0, pi[np.maximum(bt, 0)], -1).astype(np.int32)
    out2, lse2 = _oracle_f64(q, kc2, vc2, bt2, n, 0.4)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


def test_shared_blocks_equal_private_copies_bitwise():
    # Two requests share their first two physical blocks, as in the
    # stanleyjacob.dev "vLLM" walkthrough, Part V "PagedAttention and the KV
    # block manager" (tables A: 0->7, 1->2, 2->9 and B: 0->7, 1->2, 2->4).
    rng = np.random.default_rng(9)
    Hkv, d, bs = 2, 8, 16
    prefix_K = rng.standard_normal((32, Hkv, d))
    prefix_V = rng.standard_normal((32, Hkv, d))
    tails = [rng.standard_normal((10, Hkv, d)) for _ in range(4)]
    KA = np.concatenate([prefix_K, tails[0]])
    VA = np.concatenate([prefix_V, tails[1]])
    KB = np.concatenate([prefix_K, tails[2]])
    VB = np.concatenate([prefix_V, tails[3]])
    q = rng.standard_normal((2, 4, d))
    NB = 10
    kc = np.full((NB, bs, Hkv, d), np.nan)
    vc = kc.copy()
    kc[7], vc[7] = prefix_K[:16], prefix_V[:16]
    kc[2], vc[2] = prefix_K[16:], prefix_V[16:]
    kc[9, :10], vc[9, :10] = tails[0], tails[1]
    kc[4, :10], vc[4, :10] = tails[2], tails[3]
    bt_shared = np.array([[7, 2, 9], [7, 2, 4]], np.int32)
    n = np.array([42, 42], np.int32)
    shared_out, shared_lse = _oracle_f64(q, kc, vc, bt_shared, n, 0.35)
    # Private copies of the prefix for B.
    kc[0], vc[0] = prefix_K[:16], prefix_V[:16]
    kc[1], vc[1] = prefix_K[16:], prefix_V[16:]
    bt_private = np.array([[7, 2, 9], [0, 1, 4]], np.int32)
    priv_out, priv_lse = _oracle_f64(q, kc, vc, bt_private, n, 0.35)
    np.testing.assert_array_equal(shared_out, priv_out)
    np.testing.assert_array_equal(shared_lse, priv_lse)
    for i, (K, V) in enumerate([(KA, VA), (KB, VB)]):
        bo, _ = brute_attention(q[i], K, V, 0.35)
        np.testing.assert_allclose(shared_out[i], bo, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- c-iv..c-vii closed forms
def test_single_token_returns_value_row_exactly():
    rng = np.random.default_rng(1)
    q, Ks, Vs = rand_case(rng, 2, 4, 2, 8, [1, 1])
    kc, vc, bt, n = scatter_into_pool(Ks, Vs, 8, 16, rng)
    out, lse = _oracle_f64(q, kc, vc, bt, n, 0.5)
    for i in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[i, h], Vs[i][0, h // 2])
            s = 0.5 * float(np.dot(q[i, h], Ks[i][0, h // 2]))
            assert lse[i, h] == pytest.approx(s, abs=1e-14)


def test_one_hot_logits_select_marked_row_exactly():
    rng = np.random.default_rng(4)
    Hq, Hkv, d, n = 4, 2, 8, 50
    q = rng.standard_normal((1, Hq, d))
    for star in [0, 15, 16, 31, 49]:
        K = np.zeros((n, Hkv, d))
        for kvh in range(Hkv):
            K[star, kvh] = 1e3 * q[0, kvh * 2:(kvh + 1) * 2].mean(axis=0)
        V = rng.standard_normal((n, Hkv, d))
        kc, vc, bt, nn = scatter_into_pool([K], [V], 8, 16, rng)
        out, _ = _oracle_f64(q, kc, vc, bt, nn, 1.0)
        for h in range(Hq):
            np.testing.assert_array_equal(out[0, h], V[star, h // 2])


def test_uniform_weights_give_mean_and_log_n():
    rng = np.random.default_rng(6)
    Hq, Hkv, d = 4, 4, 8
    for n in [1, 7, 16, 33]:
        q = np.zeros((1, Hq, d))
        K = rng.standard_normal((n, Hkv, d))
        V = rng.standard_normal((n, Hkv, d))
        kc, vc, bt, nn = scatter_into_pool([K], [V], 8, 16, rng)
        out, lse = _oracle_f64(q, kc, vc, bt, nn, 0.7)
        np.testing.assert_allclose(out[0], V.mean(axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0], math.log(n), rtol=0, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(8)
    Hq, Hkv, d, n = 8, 2, 8, 23
    g = Hq // Hkv
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((n, Hkv, d))
    V = rng.standard_normal((n, Hkv, d))
    o_gqa, l_gqa = oracle.attention_contiguous(q, K, V, 0.3)
    o_mha, l_mha = oracle.attention_contiguous(q, np.repeat(K, g, axis=1), np.repeat(V, g, axis=1), 0.3)
    np.testing.assert_allclose(o_gqa, o_mha, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l_gqa, l_mha, rtol=0, atol=1e-14)
    # Head h must read kv head h // g: moving one kv head changes exactly its g query heads.
    K2 = K.copy()
    K2[:, 1] += rng.standard_normal((n, d))  # a per-token change (a constant shift cancels in softmax)
    o2, _ = oracle.attention_contiguous(q, K2, V, 0.3)
    assert np.array_equal(o2[:g], o_gqa[:g]) and not np.allclose(o2[g:], o_gqa[g:])


def test_empty_context():
    q = np.ones((3, 4))
    out, lse = oracle.attention_contiguous(q, np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), 1.0)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_scale_and_value_roles_matter():
    rng = np.random.default_rng(10)
    q, Ks, Vs = rand_case(rng, 1, 2, 1, 4, [9])
    o1, _ = oracle.attention_contiguous(q[0], Ks[0], Vs[0], 1.0)
    o2, _ = oracle.attention_contiguous(q[0], Ks[0], Vs[0], 0.25)
    o3, _ = oracle.attention_contiguous(q[0], Vs[0], Ks[0], 1.0)
    assert not np.allclose(o1, o2) and not np.allclose(o1, o3)
    bo, _ = brute_attention(q[0], Ks[0], Vs[0], 0.25)
    np.testing.assert_allclose(o2, bo, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- c-viii LSE merge
@pytest.mark.parametrize("P", [16, 32, 512, 37])
def test_partition_merge_equals_unsplit(P):
    rng = np.random.default_rng(12)
    lens = [1, 15, 16, 100, 517]
    q, Ks, Vs = rand_case(rng, len(lens), 4, 2, 8, lens)
    kc, vc, bt, n = scatter_into_pool(Ks, Vs, 64, 16, rng)
    out, lse = _oracle_f64(q, kc, vc, bt, n, 0.3)
    num_parts = -(-max(lens) // P)
    S, Hq, d = q.shape
    op = np.zeros((S, Hq, num_parts, d))
    lp = np.full((S, Hq, num_parts), -np.inf)
    for i in range(S):
        for p in range(num_parts):
            lo, hi = p * P, min((p + 1) * P, lens[i])
            if lo < hi:
                op[i, :, p], lp[i, :, p] = brute_attention(q[i], Ks[i][lo:hi], Vs[i][lo:hi], 0.3)
    mo, ml = oracle.lse_merge(op, lp)
    np.testing.assert_allclose(mo, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)


def test_paged_decode_partitions_match_brute_force_partials():
    rng = np.random.default_rng(13)
    lens = [5, 40, 70]
    S, Hq, Hkv, d, P = 3, 4, 2, 8, 32
    qf = rng.standard_normal((S, Hq, d)).astype(np.float32)
    Ks = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in lens]
    Vs = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in lens]
    kc, vc, bt, n = scatter_into_pool(Ks, Vs, 16, 16, rng)
    kc, vc = kc.astype(np.float32), vc.astype(np.float32)
    op, lp = oracle.paged_decode_partitions(qf, kc, vc, bt, n, 0.5, "f32", P, 3)
    for i in range(S):
        for p in range(3):
            lo, hi = p * P, min((p + 1) * P, lens[i])
            if lo >= hi:
                assert np.isneginf(lp[i, :, p]).all() and (op[i, :, p] == 0).all()
                continue
            bo, bl = brute_attention(qf[i].astype(np.float64), Ks[i][lo:hi].astype(np.float64),
                                     Vs[i][lo:hi].astype(np.float64), 0.5)
            np.testing.assert_allclose(op[i, :, p], bo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lp[i, :, p], bl, rtol=0, atol=1e-12)


def test_merge_hand_computed():
    # lse_1 = 0, lse_2 = ln 3 -> weights 1/4, 3/4; total lse = ln 4.
    o = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    lp = np.array([[0.0, math.log(3.0)]])
    mo, ml = oracle.lse_merge(o, lp)
    np.testing.assert_allclose(mo, [[0.25, 0.75]], atol=1e-15)
    np.testing.assert_allclose(ml, [math.log(4.0)], atol=1e-15)


def test_merge_skips_empty_partitions_even_if_garbage():
    o = np.array([[[np.nan, np.nan], [2.0, -1.0], [np.inf, 0.0]]])
    lp = np.array([[-np.inf, 0.5, -np.inf]])
    mo, ml = oracle.lse_merge(o, lp)
    np.testing.assert_array_equal(mo, [[2.0, -1.0]])
    np.testing.assert_allclose(ml, [0.5], atol=1e-15)
    mo, ml = oracle.lse_merge(o[:, :1], lp[:, :1])
    assert (mo == 0).all() and np.isneginf(ml).all()


# ----------------------------------------------------------------- c-x reshape_and_cache
def test_reshape_writes_exactly_the_slots():
    rng = np.random.default_rng(14)
    NB, bs, Hkv, d, T = 8, 16, 2, 4, 5
    kc = np.full((NB, bs, Hkv, d), 0x7FC0, np.uint16)
    vc = kc.copy()
    key = rng.integers(0, 2 ** 16, (T, Hkv, d), dtype=np.uint16)
    val = rng.integers(0, 2 ** 16, (T, Hkv, d), dtype=np.uint16)
    slots = np.array([0, 17, -1, 127, 64], np.int64)
    k2, v2 = oracle.reshape_and_cache(key, val, kc, vc, slots, bs)
    # Independent expectation: block = slot // 16, offset = slot % 16.
    expect_k = kc.copy()
    expect_v = vc.copy()
    for t, (b, o) in enumerate([(0, 0), (1, 1), (None, None), (7, 15), (4, 0)]):
        if b is None:
            continue
        expect_k[b, o] = key[t]
        expect_v[b, o] = val[t]
    np.testing.assert_array_equal(k2, expect_k)
    np.testing.assert_array_equal(v2, expect_v)
    changed = np.any(k2.reshape(NB * bs, -1) != kc.reshape(NB * bs, -1), axis=1)
    assert changed.sum() == 4  # padding token (slot -1) writes nothing
    assert (kc == 0x7FC0).all()  # input untouched


def test_reshape_round_trip_through_gather():
    # Write tokens with the slot formula, then read them back as one-token
    # sequences through a block table: the rows come back bit-exactly.
    rng = np.random.default_rng(15)
    NB, bs, Hkv, d, T = 12, 16, 2, 8, 6
    kc = np.zeros((NB, bs, Hkv, d), np.float32)
    vc = kc.copy()
    phys = rng.choice(NB, T, replace=False)
    off = rng.integers(0, bs, T)
    slots = phys * bs + off
    key = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    val = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    k2, v2 = oracle.reshape_and_cache(key, val, kc, vc, slots, bs)
    for t in range(T):
        # A sequence whose logical block 0 is `phys`, of length off+1: its last token is slot.
        Kc, Vc = oracle.gather_context(k2, v2, np.array([phys[t]]), int(off[t]) + 1, bs)
        np.testing.assert_array_equal(Kc[-1], key[t])
        np.testing.assert_array_equal(Vc[-1], val[t])
