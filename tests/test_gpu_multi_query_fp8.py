"""GPU parity for the multi-query kernel over FP8 (E4M3) caches: pa_multi_query_fp8
against the oracle's multi-query attention on code values times the scales, and
the one-token-per-sequence path of pa_decode_fp8 through the same kernel."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_TOL, TOL, ensure_built, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _fp8_case(Hq, Hkv, d, qlens, nlens, seed):
    base = W.small_case("mq8", len(qlens), Hq, Hkv, d, "bf16", ("uniform", 1, 2), seed=seed, num_blocks=160,
                        kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 32)
    cfg = W.MultiQueryConfig("mq8", base, ("fixed", 1))
    return W.make_multi_inputs(cfg, context_lens=np.asarray(nlens, np.int32), query_lens=np.asarray(qlens, np.int32))


def _oracle(mq):
    """Multi-query attention over value(code) * scale: the FP8 caches read back
    in float64 and passed to the oracle as f32-typed caches."""
    p, cfg = mq.paged, mq.paged.cfg
    kc = oracle.dequantize(p.key_cache, cfg.k_scale)
    vc = oracle.dequantize(p.value_cache, cfg.v_scale)
    return oracle.paged_multi_query(mq.query, kc, vc, p.block_tables, p.context_lens, mq.query_start_loc, cfg.scale,
                                    "bf16", kv_dtype="f64")


QLENS = [1, 4, 5, 8, 9, 37, 0, 6, 2, 16, 17, 1]
NLENS = [1, 100, 16, 33, 200, 300, 50, 3, 17, 160, 17, 0]


@pytest.mark.parametrize("columns", ["16", "32"])
@pytest.mark.parametrize("d,Hq,Hkv", [(128, 32, 8), (128, 8, 8), (64, 16, 2), (64, 16, 16), (128, 12, 4)])
def test_multi_query_fp8_matches_the_oracle(pa, d, Hq, Hkv, columns):
    pa.pa_set_option(pa.PA_OPT_TILE_COLUMNS, int(columns))
    mq = _fp8_case(Hq, Hkv, d, QLENS, NLENS, seed=51)
    p, cfg = mq.paged, mq.paged.cfg
    q = to_dev(mq.query)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_multi_query_fp8(out, q, _u8(p.key_cache), _u8(p.value_cache), to_dev(p.block_tables),
                          to_dev(p.context_lens), to_dev(mq.query_start_loc), cfg.scale, cfg.k_scale, cfg.v_scale,
                          lse_out=lse)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle(mq)
    dead = np.isneginf(ref_lse)
    got, got_lse = f64(out), f64(lse)
    assert (got[dead] == 0).all() and np.isneginf(got_lse[dead]).all()
    assert np.abs(got[~dead] - ref[~dead]).max() <= TOL["bf16"]
    assert np.abs(got_lse[~dead] - ref_lse[~dead]).max() <= LSE_TOL["bf16"]


def test_fp8_decode_through_the_multi_query_kernel(pa):
    """pa_decode_fp8 with one token per sequence through the multi-query kernel
    equals the oracle's FP8 decode, empty contexts included."""
    lens = np.array([1, 15, 16, 17, 33, 100, 257, 31, 48, 129, 0], np.int32)
    for d, Hq, Hkv in [(128, 32, 8), (64, 8, 2), (128, 16, 1)]:
        cfg = W.small_case("fp8mq", len(lens), Hq, Hkv, d, "bf16", ("uniform", 1, 2), seed=52, num_blocks=220,
                           kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 32)
        inp = W.make_inputs(cfg, context_lens=np.maximum(lens, 1))
        inp.context_lens = lens
        out = torch.full((len(lens), Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((len(lens), Hq), float("nan"), dtype=torch.float32, device="cuda")
        pa.pa_decode_fp8(out, to_dev(inp.query), _u8(inp.key_cache), _u8(inp.value_cache), to_dev(inp.block_tables),
                         to_dev(lens), cfg.scale, cfg.k_scale, cfg.v_scale, lse_out=lse)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.paged_decode_fp8(inp.query, inp.key_cache, inp.value_cache, inp.block_tables, lens,
                                               cfg.scale, cfg.k_scale, cfg.v_scale)
        z = lens == 0
        assert (f64(out)[z] == 0).all() and np.isneginf(f64(lse)[z]).all()
        assert np.abs(f64(out)[~z] - ref[~z]).max() <= TOL["bf16"]
        assert np.abs(f64(lse)[~z] - ref_lse[~z]).max() <= LSE_TOL["bf16"]
