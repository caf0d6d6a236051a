"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Full-size runs of the five synthetic workloads, plus small cases that span
several tiles and ragged tails, closed forms that must hold bit-exactly, and
invariances (block placement, block sharing, run-to-run).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (LSE_TOL, PART_TOL, TOL, Dev, bits, ensure_built, f64, forced, max_err, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


@pytest.fixture(autouse=True, params=["tiles_partitions", "tiles4_pieces"])
def decode_kernel(request, pa):
    """Run every test here twice: with the tile kernel's own choice of waves
    per workgroup (8 on these small grids) and pa_decode_split cut into
    partitions on the tile kernel, then with 4-wave tile workgroups and the
    split cut into pieces on the persistent split kernel."""
    opts = dict(split_cut=1) if request.param == "tiles_partitions" else dict(tile_waves=4, split_cut=2)
    with forced(pa, **opts):
        yield request.param


def _say(msg):
    print(msg, flush=True)


# --------------------------------------------------------------- the five workloads, full size
@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_workload_reshape_then_decode(pa, cfg):
    _say(f"[{cfg.name}] generating")
    inp = W.make_inputs(cfg, mode="parity")
    kb, vb = W.caches_before_write(inp)
    d = Dev(inp, key_cache=kb, value_cache=vb)
    _say(f"[{cfg.name}] reshape_and_cache of {inp.slot_mapping.size} tokens")
    pa.pa_reshape_and_cache(to_dev(inp.new_key), to_dev(inp.new_value), d.kc, d.vc, to_dev(inp.slot_mapping))
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.reshape_and_cache(inp.new_key, inp.new_value, kb, vb, inp.slot_mapping)
    del kb, vb
    np.testing.assert_array_equal(bits(d.kc), ref_k.view(bits(d.kc[:1]).dtype))
    np.testing.assert_array_equal(bits(d.vc), ref_v.view(bits(d.vc[:1]).dtype))

    _say(f"[{cfg.name}] decode")
    out, lse = d.decode(pa, lse=True)
    out_s, lse_s, ws = d.decode_split(pa, lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.paged_decode(inp.query, ref_k, ref_v, inp.block_tables, inp.context_lens,
                                       cfg.scale, cfg.dtype)
    e1, e2 = max_err(out, ref), max_err(out_s, ref)
    l1, l2 = max_err(lse, ref_lse), max_err(lse_s, ref_lse)
    _say(f"[{cfg.name}] max|err| decode {e1:.2e} split {e2:.2e}; lse {l1:.2e} {l2:.2e}")
    assert e1 <= TOL[cfg.dtype] and e2 <= TOL[cfg.dtype]
    assert l1 <= LSE_TOL[cfg.dtype] and l2 <= LSE_TOL[cfg.dtype]

    check_split_pieces(pa, cfg, inp, ref_k, ref_v, ws, cfg.partition_size)


def check_split_pieces(pa, cfg, inp, kc, vc, ws, P, max_pairs=24):
    """The workspace partials of pa_decode_split against the oracle: pieces of
    the persistent split kernel, or P-token partitions of the tile kernel."""
    pt = pa.pa_decode_split_part_tokens(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, inp.max_context_len, P,
                                        pa.PA_DTYPE_BF16 if cfg.dtype == "bf16" else pa.PA_DTYPE_F32)
    if pt:
        return check_split_partitions(pa, cfg, inp, kc, vc, ws, P, pt, max_pairs)
    return check_pieces_cut(pa, cfg, inp, kc, vc, ws, P, max_pairs)


def check_split_partitions(pa, cfg, inp, kc, vc, ws, P, pt, max_pairs=24):
    """Slot p of (sequence i, head h) holds attention over keys
    [p*pt, min((p+1)*pt, n_i)) (pt = k * P) for every partition of a sequence
    cut in two or more (the pages' split of one context into partitions,
    merged by the log-sum-exp rule)."""
    S, Hq, Hkv, d = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_size
    g = Hq // Hkv
    o_parts, lse_parts = pa.workspace_views(ws, S, Hq, d, inp.max_context_len, P)[:2]
    go, gl = f64(o_parts), f64(lse_parts)
    q = oracle.decode_values(inp.query, cfg.dtype)
    n = inp.context_lens.astype(np.int64)
    checked = 0
    for i in range(S):
        np_i = -(-int(n[i]) // pt)
        if np_i < 2:
            continue
        Kc, Vc = oracle.gather_context(kc, vc, inp.block_tables[i], int(n[i]), 16)
        Kf, Vf = oracle.decode_values(Kc, cfg.dtype), oracle.decode_values(Vc, cfg.dtype)
        for p in sorted({0, np_i - 1, np_i // 2}):
            t0, t1 = p * pt, min((p + 1) * pt, int(n[i]))
            for h in range(Hkv):
                ro, rl = oracle.attention_contiguous(q[i, h * g:(h + 1) * g], Kf[t0:t1, h:h + 1],
                                                     Vf[t0:t1, h:h + 1], cfg.scale)
                # The tile kernel feeds the bf16 matrix cores probabilities
                # rounded to bf16 (relative error <= 2^-8 each), so a float32
                # partial may move by up to 2^-8 * max |v| over the partition.
                tol = PART_TOL[cfg.dtype]
                if cfg.dtype == "bf16":
                    tol += 2.0 ** -8 * float(np.abs(Vf[t0:t1, h]).max())
                assert np.abs(go[i, h * g:(h + 1) * g, p] - ro).max() <= tol
                assert np.abs(gl[i, h * g:(h + 1) * g, p] - rl).max() <= LSE_TOL[cfg.dtype]
        checked += 1
        if checked >= max_pairs:
            break
    return checked


def check_pieces_cut(pa, cfg, inp, kc, vc, ws, P, max_pairs=24):
    """The workspace pieces of the persistent split kernel against the oracle,
    piece by piece.

    The header gives the cut (T blocks, R ranges, per-sequence block prefix);
    kv heads go in groups of up to 8, the blocks of all sequences laid end to
    end per group. Each piece of a cut sequence must hold attention over
    exactly its token range, for every query head of its group.
    """
    S, Hq, Hkv, d = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_size
    g = Hq // Hkv
    HG = min(Hkv, 8)
    NG = -(-Hkv // HG)
    o_parts, lse_parts, T, R, prefix = pa.workspace_views(ws, S, Hq, d, inp.max_context_len, P)
    n = inp.context_lens.astype(np.int64)
    nb = (n + 15) // 16
    pre = prefix.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(pre, np.concatenate([[0], np.cumsum(nb)]))
    Tseq = int(nb.sum())
    assert T == NG * Tseq and 1 <= R <= max(1, T // (P // 16))
    rng_of = lambda x: (x * R + R - 1) // T  # noqa: E731
    go, gl = f64(o_parts), f64(lse_parts)
    q = oracle.decode_values(inp.query, cfg.dtype)
    checked = 0
    for i in range(S):
        if nb[i] == 0:
            continue
        for gi in range(NG):
            x0 = gi * Tseq + int(pre[i])
            r0, r1 = rng_of(x0), rng_of(x0 + int(nb[i]) - 1)
            if r0 == r1:
                continue
            Kc, Vc = oracle.gather_context(kc, vc, inp.block_tables[i], int(n[i]), 16)
            Kf, Vf = oracle.decode_values(Kc, cfg.dtype), oracle.decode_values(Vc, cfg.dtype)
            for r in range(r0, r1 + 1):
                lo = max(x0, r * T // R) - x0
                hi = min(x0 + int(nb[i]), (r + 1) * T // R) - x0
                assert hi - lo >= 1
                t0, t1 = lo * 16, min(hi * 16, int(n[i]))
                j = r - r0
                for h in range(gi * HG, min(Hkv, (gi + 1) * HG)):
                    ro, rl = oracle.attention_contiguous(q[i, h * g:(h + 1) * g], Kf[t0:t1, h:h + 1],
                                                         Vf[t0:t1, h:h + 1], cfg.scale)
                    assert np.abs(go[i, h * g:(h + 1) * g, j] - ro).max() <= PART_TOL[cfg.dtype]
                    assert np.abs(gl[i, h * g:(h + 1) * g, j] - rl).max() <= LSE_TOL[cfg.dtype]
            checked += 1
            if checked >= max_pairs:
                return checked
    return checked


# --------------------------------------------------------------- shape sweep, ragged tails
SWEEP = []
for dtype in ("f32", "bf16"):
    for d_h in (64, 128):
        for Hq, Hkv in ((2, 2), (4, 2), (6, 2), (8, 2), (16, 2), (32, 2)):
            SWEEP.append((dtype, d_h, Hq, Hkv))


@pytest.mark.parametrize("dtype,d_h,Hq,Hkv", SWEEP, ids=lambda v: str(v))
def test_shape_sweep(pa, dtype, d_h, Hq, Hkv):
    lens = np.array([1, 15, 16, 17, 33, 100, 257, 31, 48, 129], np.int32)
    cfg = W.small_case("sweep", len(lens), Hq, Hkv, d_h, dtype, ("uniform", 1, 2), seed=21,
                       num_blocks=200, partition_size=32)
    inp = W.make_inputs(cfg, context_lens=lens)
    d = Dev(inp)
    out, lse = d.decode(pa, lse=True)
    outs = [d.decode_split(pa, partition_size=P, lse=True)[:2] for P in (16, 32, 64, 512)]
    torch.cuda.synchronize()
    ref, ref_lse = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                       inp.context_lens, cfg.scale, dtype)
    assert max_err(out, ref) <= TOL[dtype]
    assert max_err(lse, ref_lse) <= LSE_TOL[dtype]
    for o, l in outs:
        assert max_err(o, ref) <= TOL[dtype]
        assert max_err(l, ref_lse) <= LSE_TOL[dtype]


def _split_long_contexts(pa, Hq, Hkv):
    cfg = W.small_case("pieces", 5, Hq, Hkv, 128, "bf16", ("uniform", 900, 3000), seed=31, num_blocks=1200,
                       partition_size=64)
    inp = W.make_inputs(cfg)
    d = Dev(inp)
    for P in (16, 64, 256):
        out, lse, ws = d.decode_split(pa, partition_size=P, lse=True)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                           inp.context_lens, cfg.scale, cfg.dtype)
        assert max_err(out, ref) <= TOL["bf16"] and max_err(lse, ref_lse) <= LSE_TOL["bf16"]
        assert check_split_pieces(pa, cfg, inp, inp.key_cache, inp.value_cache, ws, P, max_pairs=8) >= 1


@pytest.mark.parametrize("Hq,Hkv", [(16, 4), (24, 12)])
def test_split_pieces_long_contexts(pa, decode_kernel, Hq, Hkv):
    """Long contexts cut in many pieces or partitions (partitions of k * P
    tokens, k the library's choice)."""
    _split_long_contexts(pa, Hq, Hkv)


@pytest.mark.parametrize("factor", [1, 3])
@pytest.mark.parametrize("Hq,Hkv", [(16, 4), (24, 12)])
def test_split_partition_factor_forced(pa, Hq, Hkv, factor):
    """The partition cut with its factor forced: partitions of P and 3 * P tokens."""
    pa.pa_set_option(pa.PA_OPT_SPLIT_CUT, 1)
    pa.pa_set_option(pa.PA_OPT_SPLIT_PART_FACTOR, factor)
    _split_long_contexts(pa, Hq, Hkv)


# --------------------------------------------------------------- closed forms, bit-exact
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_context_is_the_value_row(pa, dtype):
    cfg = W.small_case("one", 12, 8, 2, 128, dtype, ("uniform", 1, 2), seed=5, num_blocks=64)
    inp = W.make_inputs(cfg, context_lens=np.ones(12, np.int32))
    d = Dev(inp)
    out, _ = d.decode(pa)
    out_s, _, _ = d.decode_split(pa, partition_size=16)
    torch.cuda.synchronize()
    g = cfg.group
    expect = np.stack([np.repeat(inp.new_value[i], g, axis=0) for i in range(12)])  # V at position 0
    np.testing.assert_array_equal(bits(out), expect.view(bits(out[:1]).dtype))
    np.testing.assert_array_equal(bits(out_s), expect.view(bits(out[:1]).dtype))


def _one_hot_inputs(dtype, star_positions, seed=7):
    S = len(star_positions)
    lens = np.array([max(p + 1 + (i * 37) % 200, p + 1) for i, p in enumerate(star_positions)], np.int32)
    cfg = W.small_case("onehot", S, 8, 2, 128, dtype, ("uniform", 1, 2), seed=seed, num_blocks=400,
                       partition_size=64)
    inp = W.make_inputs(cfg, context_lens=lens)
    # Positive queries; keys zero except one marked token per (sequence, kv head)
    # equal to 16 * ones: its logit is 16 * sum|q| * scale, every other is 0, so
    # all other weights are exactly 0 in float32 and the output is V at the mark.
    q = np.abs(W.bf16_bits_to_f32(inp.query) if dtype == "bf16" else inp.query)
    inp.query = W.f32_to_bf16_bits(q) if dtype == "bf16" else q.astype(np.float32)
    kz = np.zeros_like(inp.key_cache)
    big = np.float32(16.0)
    mark = W.f32_to_bf16_bits(np.array([big], np.float32))[0] if dtype == "bf16" else big
    expect = np.zeros((S, cfg.num_heads, cfg.head_size), dtype=inp.value_cache.dtype)
    for i, p in enumerate(star_positions):
        b = inp.block_tables[i, p // 16]
        kz[b, p % 16] = mark
        for h in range(cfg.num_heads):
            expect[i, h] = inp.value_cache[b, p % 16, h // cfg.group]
    # Keep the poison of unowned slots so stray reads still show.
    poison = np.isnan(W.bf16_bits_to_f32(inp.key_cache) if dtype == "bf16" else inp.key_cache)
    kz[poison] = inp.key_cache[poison]
    inp.key_cache = kz
    return cfg, inp, expect


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_hot_logits_select_the_marked_row_exactly(pa, dtype):
    stars = [0, 15, 16, 31, 32, 63, 64, 65, 127, 128, 200, 255, 256, 300]
    cfg, inp, expect = _one_hot_inputs(dtype, stars)
    d = Dev(inp)
    out, _ = d.decode(pa)
    res = [d.decode_split(pa, partition_size=P)[0] for P in (16, 64, 128)]
    torch.cuda.synchronize()
    ref, _ = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                 inp.context_lens, cfg.scale, dtype)
    ev = oracle.decode_values(expect, dtype)
    assert np.abs(ref - ev).max() <= 1e-12  # the oracle agrees with the closed form
    dt = bits(out[:1]).dtype
    np.testing.assert_array_equal(bits(out), expect.view(dt))
    for o in res:
        np.testing.assert_array_equal(bits(o), expect.view(dt))


def test_uniform_weights_give_the_mean(pa):
    cfg = W.small_case("uni", 6, 8, 2, 128, "f32", ("uniform", 1, 2), seed=9, num_blocks=200)
    lens = np.array([1, 7, 16, 33, 100, 250], np.int32)
    inp = W.make_inputs(cfg, context_lens=lens)
    inp.query = np.zeros_like(inp.query)
    d = Dev(inp)
    out, lse = d.decode(pa, lse=True)
    torch.cuda.synchronize()
    for i, n in enumerate(lens):
        Kc, Vc = oracle.gather_context(inp.key_cache, inp.value_cache, inp.block_tables[i], int(n), 16)
        mean = np.repeat(Vc.astype(np.float64).mean(axis=0), cfg.group, axis=0)
        assert np.abs(f64(out)[i] - mean).max() <= 1e-5
        assert np.abs(f64(lse)[i] - math.log(n)).max() <= 1e-5


# --------------------------------------------------------------- invariances, bit-exact
def test_block_permutation_invariance(pa):
    cfg = W.small_case("perm", 8, 32, 8, 128, "bf16", ("uniform", 20, 400), seed=11, num_blocks=300)
    inp = W.make_inputs(cfg)
    d = Dev(inp)
    o1, _ = d.decode(pa)
    s1, _, _ = d.decode_split(pa, partition_size=64)
    pi = np.random.default_rng(3).permutation(cfg.num_blocks)
    kc2 = np.empty_like(inp.key_cache)
    vc2 = np.empty_like(inp.value_cache)
    kc2[pi] = inp.key_cache
    vc2[pi] = inp.value_cache
    inp.block_tables = np.where(inp.block_tables >= 0, pi[np.maximum(inp.block_tables, 0)], -1).astype(np.int32)
    d2 = Dev(inp, key_cache=kc2, value_cache=vc2)
    o2, _ = d2.decode(pa)
    s2, _, _ = d2.decode_split(pa, partition_size=64)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o1), bits(o2))
    np.testing.assert_array_equal(bits(s1), bits(s2))


def test_shared_prefix_equals_private_copies(pa):
    cfg = W.small_case("share", 6, 64, 8, 128, "bf16", ("prefix", 256, 10, 90), seed=13, num_blocks=400)
    inp = W.make_inputs(cfg)
    d = Dev(inp)
    o1, _ = d.decode(pa)
    # Give every sequence but the first its own copy of the shared prefix blocks.
    kc, vc, bt = inp.key_cache.copy(), inp.value_cache.copy(), inp.block_tables.copy()
    used = set(bt[bt >= 0].tolist())
    free = [b for b in range(cfg.num_blocks) if b not in used]
    for i in range(1, cfg.num_seqs):
        for j in range(inp.shared_prefix_blocks):
            nb = free.pop()
            kc[nb], vc[nb] = kc[bt[i, j]], vc[bt[i, j]]
            bt[i, j] = nb
    inp.block_tables = bt
    d2 = Dev(inp, key_cache=kc, value_cache=vc)
    o2, _ = d2.decode(pa)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o1), bits(o2))


def test_seq_order_is_only_a_schedule(pa):
    cfg = W.CONFIG_BY_NAME["llama3_8b_b64"]
    inp = W.make_inputs(cfg, mode="perf")
    d = Dev(inp)
    a, la = d.decode(pa, lse=True)
    longest_first = np.argsort(-inp.context_lens, kind="stable")
    b, lb = d.decode(pa, lse=True, seq_order=longest_first)
    c, lc = d.decode(pa, lse=True, seq_order=np.random.default_rng(1).permutation(cfg.num_seqs))
    torch.cuda.synchronize()
    for o, l in ((b, lb), (c, lc)):
        np.testing.assert_array_equal(bits(a), bits(o))
        np.testing.assert_array_equal(bits(la), bits(l))


def test_seq_order_entries_out_of_range_are_clamped(pa):
    """seq_order entries outside [0, num_seqs) are clamped to the last
    sequence (the header's contract): the listed sequences get their
    natural-order bits, the last one is written twice with the same bits, and
    the sequence no entry names keeps the caller's sentinel."""
    cfg = W.small_case("order_clamp", 24, 32, 8, 128, "bf16", ("uniform", 1, 300), seed=47, num_blocks=600)
    d = Dev(W.make_inputs(cfg))
    S = cfg.num_seqs
    want, want_lse = d.decode(pa, lse=True)
    order = np.arange(S, dtype=np.int32)
    order[S - 2], order[0], order[5] = -7, S + 5, 0  # sequence 5 is named by no entry
    order[S - 1] = 2**31 - 1
    out = torch.full_like(d.q, float("nan"))
    lse = torch.full(d.q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_decode(out, d.q, d.kc, d.vc, d.bt, d.cl, cfg.scale, lse_out=lse, seq_order=to_dev(order))
    torch.cuda.synchronize()
    named = np.ones(S, bool)
    named[[5, S - 2]] = False  # S - 2 is listed only through clamped entries, which name S - 1
    np.testing.assert_array_equal(bits(out)[named], bits(want)[named])
    np.testing.assert_array_equal(bits(lse)[named], bits(want_lse)[named])
    for i in (5, S - 2):
        assert np.isnan(f64(out)[i]).all() and np.isnan(f64(lse)[i]).all()


def test_many_jobs_per_workgroup(pa):
    """Far more (sequence, kv head) jobs than resident workgroups: many rounds
    of tile workgroups, short and empty jobs included, and the schedule
    (natural order, longest first, random) never changes a bit."""
    S = 1100
    cfg = W.small_case("many_jobs", S, 16, 8, 64, "bf16", ("uniform", 1, 40), seed=41, num_blocks=4000)
    inp = W.make_inputs(cfg)
    lens = inp.context_lens.copy()
    lens[::7] = 0
    inp.context_lens = lens
    d = Dev(inp)
    _say(f"many_jobs: {S * cfg.num_kv_heads} jobs")
    a, la = d.decode(pa, lse=True)
    others = [d.decode(pa, lse=True, seq_order=np.argsort(-lens, kind="stable")),
              d.decode(pa, lse=True, seq_order=np.random.default_rng(2).permutation(S))]
    torch.cuda.synchronize()
    ref, ref_lse = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                       lens, cfg.scale, "bf16")
    assert max_err(a, ref) <= TOL["bf16"] and max_err(la, ref_lse) <= LSE_TOL["bf16"]
    assert (f64(a)[lens == 0] == 0).all() and np.isneginf(f64(la)[lens == 0]).all()
    for o, l in others:
        np.testing.assert_array_equal(bits(a), bits(o))
        np.testing.assert_array_equal(bits(la), bits(l))


def test_run_to_run_deterministic(pa):
    cfg = W.CONFIG_BY_NAME["prefix_70b"]
    inp = W.make_inputs(cfg, mode="perf")
    d = Dev(inp)
    a, _ = d.decode(pa)
    b, _ = d.decode(pa)
    c, _, _ = d.decode_split(pa)
    e, _, _ = d.decode_split(pa)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(a), bits(b))
    np.testing.assert_array_equal(bits(c), bits(e))


# --------------------------------------------------------------- edge cases
def test_empty_contexts(pa):
    lens = np.array([0, 5, 0, 40], np.int32)
    cfg = W.small_case("empty", 4, 8, 2, 64, "f32", ("uniform", 1, 2), seed=1, num_blocks=32)
    inp = W.make_inputs(cfg, context_lens=np.maximum(lens, 1))
    inp.context_lens = lens
    d = Dev(inp)
    out, lse = d.decode(pa, lse=True)
    out_s, lse_s, _ = d.decode_split(pa, partition_size=16, lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                       lens, cfg.scale, "f32")
    for o, l in ((out, lse), (out_s, lse_s)):
        assert (f64(o)[lens == 0] == 0).all() and np.isneginf(f64(l)[lens == 0]).all()
        assert max_err(o, ref) <= 1e-5 and max_err(l, ref_lse) <= 1e-5


@pytest.mark.parametrize("rows", ["1", "2", "4"])
@pytest.mark.parametrize("P", [9, 40, 70, 130])
def test_merge_partitions_alone(pa, P, rows):
    """One batch of partials (9), two (40), the lane-strided log-sum-exps past
    64 (70, 130); 30 rows (a ragged last workgroup at 4 rows each)."""
    pa.pa_set_option(pa.PA_OPT_MERGE_ROWS, int(rows))
    rng = np.random.default_rng(17)
    S, H, dh = 5, 6, 128
    o = rng.standard_normal((S, H, P, dh)).astype(np.float32)
    lp = (rng.standard_normal((S, H, P)) * 3).astype(np.float32)
    lp[rng.random((S, H, P)) < 0.3] = -np.inf
    lp[0, 0, :] = -np.inf          # a row with no context at all
    o[np.isneginf(lp)] = np.nan    # never read
    for dtype in ("f32", "bf16"):
        out = torch.empty((S, H, dh), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
        lse = torch.empty((S, H), dtype=torch.float32, device="cuda")
        pa.pa_merge_partitions(out, to_dev(o), to_dev(lp), lse_out=lse)
        torch.cuda.synchronize()
        ro, rl = oracle.lse_merge(o.astype(np.float64), lp.astype(np.float64))
        assert max_err(out, ro) <= TOL[dtype] and max_err(lse, rl) <= 1e-5


def test_reshape_skips_padding_and_out_of_range_slots(pa):
    NB, Hkv, dh, T = 16, 2, 64, 6
    kc = torch.full((NB, 16, Hkv, dh), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = kc.clone()
    rng = np.random.default_rng(2)
    key = W.f32_to_bf16_bits(rng.standard_normal((T, Hkv, dh)).astype(np.float32))
    val = W.f32_to_bf16_bits(rng.standard_normal((T, Hkv, dh)).astype(np.float32))
    slots = np.array([3, -1, 255, 256, 100000, 17], np.int64)
    before_k, before_v = bits(kc), bits(vc)
    pa.pa_reshape_and_cache(to_dev(key), to_dev(val), kc, vc, to_dev(slots))
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(key, val, before_k, before_v, slots)
    np.testing.assert_array_equal(bits(kc), ek)
    np.testing.assert_array_equal(bits(vc), ev)


def test_bad_table_entries_never_fault(pa):
    # Contents are the caller's contract; out-of-range ids are clamped, so the
    # call completes (numbers unspecified) instead of reading outside the pool.
    cfg = W.small_case("bad", 3, 8, 2, 128, "bf16", ("uniform", 40, 60), seed=4, num_blocks=16)
    inp = W.make_inputs(cfg)
    inp.block_tables[:, 1] = np.array([-5, 10 ** 6, 2 ** 31 - 1], np.int32)
    inp.context_lens = np.array([50, 10 ** 6, -3], np.int32)
    d = Dev(inp)
    out, _ = d.decode(pa)
    out_s, _, _ = d.decode_split(pa, partition_size=16, max_context_len=64)
    torch.cuda.synchronize()
    assert out.shape == out_s.shape
