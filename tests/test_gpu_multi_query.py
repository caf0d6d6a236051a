"""GPU parity for pa_multi_query against the oracle's multi-query attention:
small sweeps over head shapes and mixes of new-token counts (both tile widths),
the degenerate cases, invariance under block placement, the write-then-attend
step, and the full-size workloads on every row."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_TOL, TOL, bits, ensure_built, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


def _run(pa, mq, kc=None, vc=None, bt=None, lse=True):
    p = mq.paged
    q = to_dev(mq.query)
    out = torch.full_like(q, float("nan"))
    lse_t = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda") if lse else None
    pa.pa_multi_query(out, q, to_dev(p.key_cache if kc is None else kc), to_dev(p.value_cache if vc is None else vc),
                      to_dev(p.block_tables if bt is None else bt), to_dev(p.context_lens),
                      to_dev(mq.query_start_loc), p.cfg.scale, lse_out=lse_t)
    torch.cuda.synchronize()
    return out, lse_t


def _check(mq, out, lse, rows=None):
    p = mq.paged
    dt = p.cfg.dtype
    loc = mq.query_start_loc
    if rows is None:
        ref, ref_lse = oracle.paged_multi_query(mq.query, p.key_cache, p.value_cache, p.block_tables,
                                                p.context_lens, loc, p.cfg.scale, dt)
        got, got_lse = f64(out), f64(lse)
    else:
        ref, ref_lse, got, got_lse = _sampled_reference(mq, rows, out, lse)
    dead = np.isneginf(ref_lse)
    assert (got[dead] == 0).all() and np.isneginf(got_lse[dead]).all()
    assert np.isfinite(got[~dead]).all()
    assert np.abs(got[~dead] - ref[~dead]).max(initial=0) <= TOL[dt]
    assert np.abs(got_lse[~dead] - ref_lse[~dead]).max(initial=0) <= LSE_TOL[dt]


def _sampled_reference(mq, rows, out, lse):
    """Oracle rows for a sample of token rows (each a decode of its prefix)."""
    p = mq.paged
    loc = mq.query_start_loc
    seq_of = np.searchsorted(loc, rows, side="right") - 1
    ref = np.zeros((len(rows),) + mq.query.shape[1:])
    ref_lse = np.zeros((len(rows), mq.query.shape[1]))
    for k, (t, i) in enumerate(zip(rows, seq_of)):
        n, q = int(p.context_lens[i]), int(mq.query_lens[i])
        pos = n - q + int(t - loc[i])
        o1, l1 = oracle.paged_decode(mq.query[t:t + 1], p.key_cache, p.value_cache, p.block_tables[i:i + 1],
                                     np.array([pos + 1]), p.cfg.scale, p.cfg.dtype)
        ref[k], ref_lse[k] = o1[0], l1[0]
    return ref, ref_lse, f64(out)[rows], f64(lse)[rows]


def _case(d, Hq, Hkv, dtype, qlens, nlens, seed=31):
    base = W.small_case("mq", len(qlens), Hq, Hkv, d, dtype, ("uniform", 1, 2), seed=seed, num_blocks=160)
    cfg = W.MultiQueryConfig("mq", base, ("fixed", 1))
    return W.make_multi_inputs(cfg, context_lens=np.asarray(nlens, np.int32), query_lens=np.asarray(qlens, np.int32))


# New-token counts around the tile widths (16 or 32 columns = 16/g or 32/g
# tokens), a long prompt chunk, a sequence with no new token, one with more new
# tokens than stored ones, and an empty context.
QLENS = [1, 4, 5, 8, 9, 37, 0, 6, 2, 16, 17, 1]
NLENS = [1, 100, 16, 33, 200, 300, 50, 3, 17, 160, 17, 0]

SWEEP = [(d, Hq, Hkv, dt) for dt in ("bf16", "f32") for d in (64, 128)
         for Hq, Hkv in ((8, 8), (8, 4), (8, 2), (16, 4), (16, 2), (16, 1), (6, 2))]


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("columns", ["16", "32", "auto"])
@pytest.mark.parametrize("d,Hq,Hkv,dtype", SWEEP, ids=lambda v: str(v))
def test_multi_query_matches_the_oracle(pa, d, Hq, Hkv, dtype, columns, waves):
    """Both workgroup sizes (fp32 caches and 32-column tiles always run 4 waves)."""
    if columns != "auto":
        pa.pa_set_option(pa.PA_OPT_TILE_COLUMNS, int(columns))
    pa.pa_set_option(pa.PA_OPT_TILE_WAVES, int(waves))
    mq = _case(d, Hq, Hkv, dtype, QLENS, NLENS)
    out, lse = _run(pa, mq)
    _check(mq, out, lse)


def test_one_token_each_matches_decode_oracle(pa):
    lens = np.array([1, 15, 16, 17, 33, 100, 257, 31], np.int32)
    mq = _case(128, 32, 8, "bf16", np.ones(8, np.int32), lens, seed=33)
    out, lse = _run(pa, mq)
    ref, ref_lse = oracle.paged_decode(mq.query, mq.paged.key_cache, mq.paged.value_cache, mq.paged.block_tables,
                                       lens, mq.paged.cfg.scale, "bf16")
    assert np.abs(f64(out) - ref).max() <= TOL["bf16"]
    assert np.abs(f64(lse) - ref_lse).max() <= LSE_TOL["bf16"]


def test_batch_order_does_not_change_rows(pa):
    """The same step with its sequences listed in another order (the bench
    lists them longest context first): every sequence's rows are bit-identical,
    for both tile widths and both workgroup sizes of the 16-column tiles."""
    mq = _case(128, 32, 8, "bf16", QLENS, NLENS, seed=37)
    order = np.random.default_rng(6).permutation(len(QLENS))
    r = W.reorder_multi_inputs(mq, order)
    rows = np.concatenate([np.arange(mq.query_start_loc[i], mq.query_start_loc[i + 1]) for i in order])
    for columns in (16, 32):
        for waves in (4, 8):
            pa.pa_set_option(pa.PA_OPT_TILE_COLUMNS, columns)
            pa.pa_set_option(pa.PA_OPT_TILE_WAVES, waves)
            a, la = _run(pa, mq)
            b, lb = _run(pa, r)
            np.testing.assert_array_equal(bits(a)[rows], bits(b))
            np.testing.assert_array_equal(bits(la)[rows], bits(lb))


def test_block_placement_does_not_change_bits(pa):
    mq = _case(128, 32, 8, "bf16", QLENS, NLENS, seed=34)
    a, la = _run(pa, mq)
    p = mq.paged
    perm = np.random.default_rng(5).permutation(p.cfg.num_blocks)
    inv = np.argsort(perm)
    bt = np.where(p.block_tables >= 0, inv[np.maximum(p.block_tables, 0)], -1).astype(np.int32)
    b, lb = _run(pa, mq, kc=p.key_cache[perm], vc=p.value_cache[perm], bt=bt)
    np.testing.assert_array_equal(bits(a), bits(b))
    np.testing.assert_array_equal(bits(la), bits(lb))


def test_write_then_attend(pa):
    """pa_reshape_and_cache of every new token into a pool where their slots
    hold NaN, then pa_multi_query: equal to attending over the complete caches."""
    mq = _case(128, 32, 8, "bf16", [5, 5, 1, 12, 5], [40, 5, 90, 12, 300], seed=35)
    kc_h, vc_h = W.multi_caches_before_write(mq)
    kc, vc = to_dev(kc_h), to_dev(vc_h)
    pa.pa_reshape_and_cache(to_dev(mq.new_key), to_dev(mq.new_value), kc, vc, to_dev(mq.slot_mapping))
    np.testing.assert_array_equal(bits(kc), mq.paged.key_cache)
    out, lse = _run(pa, mq, kc=bits(kc), vc=bits(vc))
    _check(mq, out, lse)


def test_no_lse_and_host_errors(pa):
    mq = _case(64, 8, 2, "bf16", [3, 1], [10, 20], seed=36)
    out, lse = _run(pa, mq, lse=False)
    assert lse is None and np.isfinite(f64(out)).all()
    q = to_dev(mq.query)
    p = mq.paged
    args = (to_dev(p.key_cache), to_dev(p.value_cache), to_dev(p.block_tables), to_dev(p.context_lens))
    with pytest.raises(ValueError):
        pa.pa_multi_query(torch.empty_like(q), q, *args, to_dev(mq.query_start_loc[:-1]), p.cfg.scale)
    with pytest.raises(pa.PaError):
        pa.pa_multi_query(torch.empty_like(q), q, *args, to_dev(mq.query_start_loc), -1.0)


@pytest.mark.parametrize("name", [c.name for c in W.MQ_CONFIGS])
def test_full_size_workloads(pa, name):
    """The benchmarked steps at full size: every row against the oracle."""
    cfg = W.MQ_CONFIG_BY_NAME[name]
    mq = W.make_multi_inputs(cfg, mode="perf")
    out, lse = _run(pa, mq)
    assert np.isfinite(f64(out)).all() and np.isfinite(f64(lse)).all()
    _check(mq, out, lse)
