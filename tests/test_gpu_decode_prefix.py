"""GPU parity for pa_decode_prefix (shared-prefix decode: one pass over the
shared blocks for all queries, one over each sequence's own blocks, exact
log-sum-exp merge) against the oracle's decode."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_TOL, TOL, Dev, bits, ensure_built, f64, forced, to_dev

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


def _prefix_decode(pa, dev, prefix_blocks, lse=True, order=None):
    S, Hq, d = dev.q.shape
    ws = torch.empty(pa.pa_decode_prefix_workspace_bytes(S, Hq, d), dtype=torch.uint8, device="cuda")
    out = torch.full_like(dev.q, float("nan"))
    lse_t = torch.full((S, Hq), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    pa.pa_decode_prefix(out, dev.q, dev.kc, dev.vc, dev.bt, dev.cl, dev.cfg.scale, prefix_blocks, ws,
                        lse_out=lse_t, seq_order=order)
    torch.cuda.synchronize()
    return out, lse_t


def _check(inp, out, lse):
    ref, ref_lse = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                       inp.context_lens, inp.cfg.scale, inp.cfg.dtype)
    dt = inp.cfg.dtype
    assert np.abs(f64(out) - ref).max() <= TOL[dt]
    assert np.abs(f64(lse) - ref_lse).max() <= LSE_TOL[dt]


CASES = [(d, Hq, Hkv, dt, P) for dt in ("bf16", "f32") for d in (64, 128)
         for Hq, Hkv in ((64, 8), (8, 2), (16, 16), (12, 4)) for P in (1, 3, 9)]


@pytest.mark.parametrize("d,Hq,Hkv,dtype,P", CASES, ids=lambda v: str(v))
def test_prefix_decode_matches_the_oracle(pa, d, Hq, Hkv, dtype, P):
    lens = P * 16 + np.array([0, 1, 15, 16, 17, 100, 3, 64, 0, 250, 33], np.int32)
    cfg = W.small_case("prefix", len(lens), Hq, Hkv, d, dtype, ("prefix", P * 16, 0, 1), seed=41, num_blocks=160)
    inp = W.make_inputs(cfg, context_lens=lens)
    out, lse = _prefix_decode(pa, Dev(inp), P)
    _check(inp, out, lse)


@pytest.mark.parametrize("P", [3, 9, 16])
def test_sequences_shorter_than_the_prefix(pa, P):
    """Contexts that end inside the shared blocks (in any of its key ranges)
    see only their own tokens."""
    k = P * 16
    lens = np.array([k, 5, 16, 31, k - 1, k + 12, 1, k // 2, k // 2 + 1, 80, 81, 0], np.int32)
    cfg = W.small_case("prefix", len(lens), 32, 8, 128, "bf16", ("prefix", k, 0, 1), seed=42, num_blocks=60)
    inp = W.make_inputs(cfg, mode="perf", context_lens=np.maximum(lens, k))
    inp.context_lens = lens
    out, lse = _prefix_decode(pa, Dev(inp), P)
    _check_allow_empty(inp, out, lse)


def _check_allow_empty(inp, out, lse):
    ref, ref_lse = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                       inp.context_lens, inp.cfg.scale, inp.cfg.dtype)
    dead = inp.context_lens == 0
    assert (f64(out)[dead] == 0).all() and np.isneginf(f64(lse)[dead]).all()
    assert np.abs(f64(out)[~dead] - ref[~dead]).max() <= TOL["bf16"]
    assert np.abs(f64(lse)[~dead] - ref_lse[~dead]).max() <= LSE_TOL["bf16"]


def test_zero_prefix_is_pa_decode(pa):
    cfg = W.small_case("prefix", 9, 32, 8, 128, "bf16", ("prefix", 32, 1, 200), seed=43, num_blocks=140)
    dev = Dev(W.make_inputs(cfg))
    a, la = _prefix_decode(pa, dev, 0)
    b, lb = dev.decode(pa, lse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(a), bits(b))
    np.testing.assert_array_equal(bits(la), bits(lb))


def test_schedule_and_placement_do_not_change_bits(pa):
    cfg = W.small_case("prefix", 20, 64, 8, 128, "bf16", ("prefix", 64, 1, 300), seed=44, num_blocks=300)
    inp = W.make_inputs(cfg)
    dev = Dev(inp)
    a, la = _prefix_decode(pa, dev, 4)
    order = to_dev(np.argsort(-inp.context_lens, kind="stable").astype(np.int32))
    b, lb = _prefix_decode(pa, dev, 4, order=order)
    np.testing.assert_array_equal(bits(a), bits(b))
    np.testing.assert_array_equal(bits(la), bits(lb))
    perm = np.random.default_rng(3).permutation(cfg.num_blocks)
    inv = np.argsort(perm)
    moved = W.make_inputs(cfg)
    moved.key_cache, moved.value_cache = inp.key_cache[perm], inp.value_cache[perm]
    moved.block_tables = np.where(inp.block_tables >= 0, inv[np.maximum(inp.block_tables, 0)], -1).astype(np.int32)
    c, lc = _prefix_decode(pa, Dev(moved), 4)
    np.testing.assert_array_equal(bits(a), bits(c))
    np.testing.assert_array_equal(bits(la), bits(lc))


def test_workspace_and_argument_errors(pa):
    cfg = W.small_case("prefix", 3, 8, 2, 64, "bf16", ("prefix", 32, 1, 20), seed=45, num_blocks=40)
    dev = Dev(W.make_inputs(cfg))
    S, Hq, d = dev.q.shape
    out = torch.empty_like(dev.q)
    small = torch.empty(pa.pa_decode_prefix_workspace_bytes(S, Hq, d) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_prefix(out, dev.q, dev.kc, dev.vc, dev.bt, dev.cl, cfg.scale, 2, small)
    assert e.value.status == 3
    ws = torch.empty(pa.pa_decode_prefix_workspace_bytes(S, Hq, d), dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PaError):
        pa.pa_decode_prefix(out, dev.q, dev.kc, dev.vc, dev.bt, dev.cl, cfg.scale, dev.bt.shape[1] + 1, ws)


def test_prefix_70b_full_size(pa):
    """The 70B-shaped shared-prefix workload at full size: every row of the
    shared-prefix decode against the oracle, and against pa_decode."""
    cfg = W.CONFIG_BY_NAME["prefix_70b"]
    inp = W.make_inputs(cfg)
    dev = Dev(inp)
    out, lse = _prefix_decode(pa, dev, inp.shared_prefix_blocks)
    ref_out, ref_lse = dev.decode(pa, lse=True)
    torch.cuda.synchronize()
    assert np.abs(f64(out) - f64(ref_out)).max() <= TOL["bf16"]
    assert np.abs(f64(lse) - f64(ref_lse)).max() <= LSE_TOL["bf16"]
    ref, rl = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables, inp.context_lens,
                                  cfg.scale, "bf16")
    assert np.abs(f64(out) - ref).max() <= TOL["bf16"]
    assert np.abs(f64(lse) - rl).max() <= LSE_TOL["bf16"]
