"""GPU parity for pa_multi_query_split against the oracle's multi-query
attention: sweeps over head shapes, tile widths, workgroup sizes and partition
sizes on a mix of new-token counts (empty contexts, more new tokens than stored
keys, chunks longer than a partition), the workspace partials against the
oracle over each partition's keys, invariance under block placement, host
errors, and the two full-size multi-query workloads on sampled rows."""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_TOL, PART_TOL, TOL, bits, ensure_built, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


def _case(d, Hq, Hkv, dtype, qlens, nlens, seed=41):
    base = W.small_case("mqs", len(qlens), Hq, Hkv, d, dtype, ("uniform", 1, 2), seed=seed, num_blocks=160)
    cfg = W.MultiQueryConfig("mqs", base, ("fixed", 1))
    return W.make_multi_inputs(cfg, context_lens=np.asarray(nlens, np.int32), query_lens=np.asarray(qlens, np.int32))


def _run(pa, mq, P, max_ctx=None, kc=None, vc=None, bt=None, lse=True, ws=None):
    p = mq.paged
    q = to_dev(mq.query)
    max_ctx = int(p.context_lens.max(initial=0)) if max_ctx is None else max_ctx
    out = torch.full_like(q, float("nan"))
    lse_t = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda") if lse else None
    if ws is None:
        nb = pa.pa_multi_query_split_workspace_bytes(mq.num_tokens, q.shape[1], q.shape[2], max_ctx, P)
        ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN partials until written
    pa.pa_multi_query_split(out, q, to_dev(p.key_cache if kc is None else kc),
                            to_dev(p.value_cache if vc is None else vc), to_dev(p.block_tables if bt is None else bt),
                            to_dev(p.context_lens), to_dev(mq.query_start_loc), p.cfg.scale, max_ctx, P, ws,
                            lse_out=lse_t)
    torch.cuda.synchronize()
    return out, lse_t, ws


def _check(mq, out, lse, rows=None):
    p = mq.paged
    dt = p.cfg.dtype
    loc = mq.query_start_loc
    if rows is None:
        ref, ref_lse = oracle.paged_multi_query(mq.query, p.key_cache, p.value_cache, p.block_tables,
                                                p.context_lens, loc, p.cfg.scale, dt)
        got, got_lse = f64(out), f64(lse)
    else:
        ref, ref_lse = _sampled_reference(mq, rows)
        got, got_lse = f64(out)[rows], f64(lse)[rows]
    dead = np.isneginf(ref_lse)
    assert (got[dead] == 0).all() and np.isneginf(got_lse[dead]).all()
    assert np.isfinite(got[~dead]).all()
    assert np.abs(got[~dead] - ref[~dead]).max(initial=0) <= TOL[dt]
    assert np.abs(got_lse[~dead] - ref_lse[~dead]).max(initial=0) <= LSE_TOL[dt]


def _position(mq, t):
    """(sequence, position) of new token t: the token at offset j of a
    sequence with n stored keys and q new tokens sits at n - q + j."""
    loc = mq.query_start_loc
    i = int(np.searchsorted(loc, t, side="right") - 1)
    return i, int(mq.paged.context_lens[i]) - int(mq.query_lens[i]) + int(t - loc[i])


def _sampled_reference(mq, rows):
    """Oracle rows for a sample of token rows (each a decode of its prefix)."""
    p = mq.paged
    ref = np.zeros((len(rows),) + mq.query.shape[1:])
    ref_lse = np.zeros((len(rows), mq.query.shape[1]))
    for k, t in enumerate(rows):
        i, pos = _position(mq, int(t))
        o1, l1 = oracle.paged_decode(mq.query[t:t + 1], p.key_cache, p.value_cache, p.block_tables[i:i + 1],
                                     np.array([max(pos + 1, 0)]), p.cfg.scale, p.cfg.dtype)
        ref[k], ref_lse[k] = o1[0], l1[0]
    return ref, ref_lse


# New-token counts around the tile widths, a chunk longer than the smallest
# partition, a sequence with no new token, one with more new tokens than
# stored keys, and an empty context.
QLENS = [1, 4, 5, 8, 9, 37, 0, 6, 2, 16, 17, 1]
NLENS = [1, 100, 16, 33, 200, 300, 50, 3, 17, 160, 17, 0]

SWEEP = [(d, Hq, Hkv, dt) for dt in ("bf16", "f32") for d in (64, 128)
         for Hq, Hkv in ((8, 8), (8, 2), (16, 4), (16, 1), (6, 2))]


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("columns", ["16", "32"])
@pytest.mark.parametrize("P", [16, 48, 128])
@pytest.mark.parametrize("d,Hq,Hkv,dtype", SWEEP, ids=lambda v: str(v))
def test_split_matches_the_oracle(pa, d, Hq, Hkv, dtype, P, columns, waves):
    pa.pa_set_option(pa.PA_OPT_TILE_COLUMNS, int(columns))
    pa.pa_set_option(pa.PA_OPT_TILE_WAVES, int(waves))
    mq = _case(d, Hq, Hkv, dtype, QLENS, NLENS)
    out, lse, _ = _run(pa, mq, P)
    _check(mq, out, lse)


@pytest.mark.parametrize("max_ctx", [300, 301, 512, 4096])
def test_max_context_len_above_the_longest(pa, max_ctx):
    """Extra workspace slots (a bound above the longest context) change nothing."""
    mq = _case(128, 32, 8, "bf16", QLENS, NLENS, seed=42)
    a, la, _ = _run(pa, mq, 64, max_ctx=300)
    b, lb, _ = _run(pa, mq, 64, max_ctx=max_ctx)
    np.testing.assert_array_equal(bits(a), bits(b))
    np.testing.assert_array_equal(bits(la), bits(lb))
    _check(mq, b, lb)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_workspace_partials(pa, dtype):
    """Slot p of (token t, head h) holds attention of that query over keys
    [p*P, min((p+1)*P, position(t) + 1)) for every slot the merge reads."""
    P = 32
    mq = _case(64, 8, 2, dtype, [1, 9, 37, 3], [90, 70, 150, 33], seed=43)
    out, lse, ws = _run(pa, mq, P)
    _check(mq, out, lse)
    p = mq.paged
    T, Hq, d = mq.query.shape
    Hkv = p.cfg.num_kv_heads
    g = Hq // Hkv
    slots = -(-int(p.context_lens.max()) // P)
    rows = T * Hq * slots
    o_parts = ws[:rows * d * 4].view(torch.float32).view(T, Hq, slots, d)
    lse_off = (rows * d * 4 + 255) // 256 * 256
    lse_parts = ws[lse_off:lse_off + rows * 4].view(torch.float32).view(T, Hq, slots)
    go, gl = f64(o_parts), f64(lse_parts)
    q = oracle.decode_values(mq.query, dtype)
    for t in range(T):
        i, pos = _position(mq, t)
        n = pos + 1
        if n <= 0:
            continue
        Kc, Vc = oracle.gather_context(p.key_cache, p.value_cache, p.block_tables[i], n, 16)
        Kf, Vf = oracle.decode_values(Kc, dtype), oracle.decode_values(Vc, dtype)
        for s in range(-(-n // P)):
            t0, t1 = s * P, min((s + 1) * P, n)
            for h in range(Hkv):
                ro, rl = oracle.attention_contiguous(q[t, h * g:(h + 1) * g], Kf[t0:t1, h:h + 1],
                                                     Vf[t0:t1, h:h + 1], p.cfg.scale)
                # bf16 probabilities feed the matrix cores (relative error
                # <= 2^-8 each): the partial may move by 2^-8 * max |v|.
                tol = PART_TOL[dtype] + (2.0 ** -8 * float(np.abs(Vf[t0:t1, h]).max()) if dtype == "bf16" else 0)
                assert np.abs(go[t, h * g:(h + 1) * g, s] - ro).max() <= tol
                assert np.abs(gl[t, h * g:(h + 1) * g, s] - rl).max() <= LSE_TOL[dtype]


def test_block_placement_and_reruns_do_not_change_bits(pa):
    mq = _case(128, 32, 8, "bf16", QLENS, NLENS, seed=44)
    a, la, ws = _run(pa, mq, 32)
    a2, la2, _ = _run(pa, mq, 32, ws=ws)                # workspace reused as the last call left it
    np.testing.assert_array_equal(bits(a), bits(a2))
    np.testing.assert_array_equal(bits(la), bits(la2))
    p = mq.paged
    perm = np.random.default_rng(6).permutation(p.cfg.num_blocks)
    inv = np.argsort(perm)
    bt = np.where(p.block_tables >= 0, inv[np.maximum(p.block_tables, 0)], -1).astype(np.int32)
    b, lb, _ = _run(pa, mq, 32, kc=p.key_cache[perm], vc=p.value_cache[perm], bt=bt)
    np.testing.assert_array_equal(bits(a), bits(b))
    np.testing.assert_array_equal(bits(la), bits(lb))


def test_tokens_outside_every_sequence_are_zero(pa):
    """query_start_loc ending before num_tokens: the trailing rows are zero with
    a log-sum-exp of -inf; the covered rows match the oracle."""
    mq = _case(64, 8, 2, "bf16", [3, 5, 4], [40, 60, 20], seed=45)
    p = mq.paged
    loc = mq.query_start_loc.copy()
    loc[-1] -= 4                                        # the last sequence keeps none of its new tokens
    q = to_dev(mq.query)
    nb = pa.pa_multi_query_split_workspace_bytes(mq.num_tokens, 8, 64, 60, 16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_multi_query_split(out, q, to_dev(p.key_cache), to_dev(p.value_cache), to_dev(p.block_tables),
                            to_dev(p.context_lens), to_dev(loc), p.cfg.scale, 60, 16, ws, lse_out=lse)
    torch.cuda.synchronize()
    assert (f64(out)[8:] == 0).all() and np.isneginf(f64(lse)[8:]).all()
    ref, ref_lse = _sampled_reference(mq, np.arange(8))
    assert np.abs(f64(out)[:8] - ref).max() <= TOL["bf16"]
    assert np.abs(f64(lse)[:8] - ref_lse).max() <= LSE_TOL["bf16"]


def test_no_lse_and_host_errors(pa):
    mq = _case(64, 8, 2, "bf16", [3, 1], [10, 20], seed=46)
    out, lse, ws = _run(pa, mq, 16, lse=False)
    assert lse is None and np.isfinite(f64(out)).all()
    q = to_dev(mq.query)
    p = mq.paged
    args = (to_dev(p.key_cache), to_dev(p.value_cache), to_dev(p.block_tables), to_dev(p.context_lens),
            to_dev(mq.query_start_loc), p.cfg.scale)
    with pytest.raises(pa.PaError):                     # partition not a multiple of the block size
        pa.pa_multi_query_split(torch.empty_like(q), q, *args, 20, 24, ws)
    with pytest.raises(pa.PaError):                     # workspace too small for the bound
        pa.pa_multi_query_split(torch.empty_like(q), q, *args, 4096, 16, ws)


@functools.lru_cache(maxsize=1)
def _full_size(name):
    """A full-size workload and the oracle's answer for every row (computed once
    per workload; the inputs are deterministic)."""
    mq = W.make_multi_inputs(W.MQ_CONFIG_BY_NAME[name], mode="perf")
    p = mq.paged
    ref, ref_lse = oracle.paged_multi_query(mq.query, p.key_cache, p.value_cache, p.block_tables, p.context_lens,
                                            mq.query_start_loc, p.cfg.scale, p.cfg.dtype)
    return mq, ref, ref_lse


@pytest.mark.parametrize("P", [256, 512])
@pytest.mark.parametrize("name", [c.name for c in W.MQ_CONFIGS])
def test_full_size_workloads(pa, name, P):
    """The benchmarked steps at full size: every row against the oracle and
    within tolerance of pa_multi_query."""
    mq, ref_o, ref_l = _full_size(name)
    loc = mq.query_start_loc
    out, lse, _ = _run(pa, mq, P)
    got, got_lse = f64(out), f64(lse)
    dead = np.isneginf(ref_l)
    assert (got[dead] == 0).all() and np.isneginf(got_lse[dead]).all()
    assert np.isfinite(got[~dead]).all()
    assert np.abs(got[~dead] - ref_o[~dead]).max(initial=0) <= TOL[mq.paged.cfg.dtype]
    assert np.abs(got_lse[~dead] - ref_l[~dead]).max(initial=0) <= LSE_TOL[mq.paged.cfg.dtype]
    p = mq.paged
    q = to_dev(mq.query)
    ref = torch.empty_like(q)
    ref_lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    pa.pa_multi_query(ref, q, to_dev(p.key_cache), to_dev(p.value_cache), to_dev(p.block_tables),
                      to_dev(p.context_lens), to_dev(loc), p.cfg.scale, lse_out=ref_lse)
    torch.cuda.synchronize()
    assert np.abs(f64(out) - f64(ref)).max() <= 2 * TOL[p.cfg.dtype]
    assert np.abs(f64(lse) - f64(ref_lse)).max() <= 2 * LSE_TOL[p.cfg.dtype]
