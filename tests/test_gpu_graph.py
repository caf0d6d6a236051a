"""The entry points under HIP graph capture (torch.cuda.graph on the current
stream): each captured call is replayed several times, with eager work (new
queries copied in) and synchronisations between the replays, and every replay
must give the bits of the same call made eagerly on the same inputs. None of
the captured calls allocates or clears memory on the host side."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import bits, ensure_built, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


def _queries(shape, dtype, n, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(shape, generator=g).to(dtype).cuda() for _ in range(n)]


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                        # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _replay_against_eager(q_static, queries, graph, outs_graph, eager):
    for r, q in enumerate(queries):
        q_static.copy_(q)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(t) for t in outs_graph]
        want = [bits(t) for t in eager(q)]
        for a, b in zip(got, want):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {r}")


def _decode_case(seed=61):
    cfg = W.small_case("graph", 48, 32, 8, 128, "bf16", ("uniform", 1, 700), seed=seed, num_blocks=2400,
                       partition_size=128)
    return cfg, W.make_inputs(cfg)


def test_reshape_and_decode_graph(pa):
    cfg, inp = _decode_case()
    kc0, vc0 = W.caches_before_write(inp)
    kc, vc = to_dev(kc0), to_dev(vc0)
    nk, nv, sm = to_dev(inp.new_key), to_dev(inp.new_value), to_dev(inp.slot_mapping)
    bt, cl = to_dev(inp.block_tables), to_dev(inp.context_lens)
    q = to_dev(inp.query)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    graph = _capture(lambda: pa.pa_reshape_and_decode(out, q, nk, nv, sm, kc, vc, bt, cl, cfg.scale, lse_out=lse))

    def eager(qr):
        kce, vce = to_dev(kc0), to_dev(vc0)
        oe, le = torch.empty_like(q), torch.empty_like(lse)
        pa.pa_reshape_and_decode(oe, qr, nk, nv, sm, kce, vce, bt, cl, cfg.scale, lse_out=le)
        torch.cuda.synchronize()
        return oe, le, kce, vce

    _replay_against_eager(q, _queries(q.shape, q.dtype, REPLAYS, 1), graph, [out, lse, kc, vc], eager)


@pytest.mark.parametrize("cut", [1, 2], ids=["partitions", "pieces"])
def test_decode_split_graph(pa, cut):
    pa.pa_set_option(pa.PA_OPT_SPLIT_CUT, cut)
    cfg, inp = _decode_case(seed=62)
    kc, vc = to_dev(inp.key_cache), to_dev(inp.value_cache)
    bt, cl = to_dev(inp.block_tables), to_dev(inp.context_lens)
    q = to_dev(inp.query)
    P = cfg.partition_size
    ws = torch.empty(pa.pa_decode_split_workspace_bytes(cfg.num_seqs, cfg.num_heads, cfg.head_size,
                                                        inp.max_context_len, P), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    graph = _capture(lambda: pa.pa_decode_split(out, q, kc, vc, bt, cl, cfg.scale, inp.max_context_len, P, ws,
                                                lse_out=lse))

    def eager(qr):
        oe, le = torch.empty_like(q), torch.empty_like(lse)
        wse = torch.empty_like(ws)
        pa.pa_decode_split(oe, qr, kc, vc, bt, cl, cfg.scale, inp.max_context_len, P, wse, lse_out=le)
        torch.cuda.synchronize()
        return oe, le

    _replay_against_eager(q, _queries(q.shape, q.dtype, REPLAYS, 2), graph, [out, lse], eager)


def test_decode_prefix_graph(pa):
    """The shared-prefix decode (its two launches and the workspace between
    them) under capture, against eager calls on fresh workspaces."""
    cfg = W.small_case("graph_prefix", 40, 64, 8, 128, "bf16", ("prefix", 96, 1, 300), seed=64, num_blocks=900)
    inp = W.make_inputs(cfg)
    kc, vc = to_dev(inp.key_cache), to_dev(inp.value_cache)
    bt, cl = to_dev(inp.block_tables), to_dev(inp.context_lens)
    q = to_dev(inp.query)
    P = inp.shared_prefix_blocks
    ws = torch.empty(pa.pa_decode_prefix_workspace_bytes(cfg.num_seqs, cfg.num_heads, cfg.head_size),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    graph = _capture(lambda: pa.pa_decode_prefix(out, q, kc, vc, bt, cl, cfg.scale, P, ws, lse_out=lse))

    def eager(qr):
        oe, le = torch.empty_like(q), torch.empty_like(lse)
        pa.pa_decode_prefix(oe, qr, kc, vc, bt, cl, cfg.scale, P, torch.empty_like(ws), lse_out=le)
        torch.cuda.synchronize()
        return oe, le

    _replay_against_eager(q, _queries(q.shape, q.dtype, REPLAYS, 4), graph, [out, lse], eager)


def test_reshape_and_decode_fp8_graph(pa):
    """The one-launch FP8 step (quantizing write and decode) under capture:
    every replay writes the same codes and gives the eager bits."""
    cfg = W.small_case("graph_fp8", 48, 32, 8, 128, "bf16", ("uniform", 1, 700), seed=65, num_blocks=2400,
                       kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 32)
    inp = W.make_inputs(cfg)
    kc0, vc0 = W.caches_before_write(inp)
    kc, vc = to_dev(kc0), to_dev(vc0)
    nk, nv, sm = to_dev(inp.new_key), to_dev(inp.new_value), to_dev(inp.slot_mapping)
    bt, cl = to_dev(inp.block_tables), to_dev(inp.context_lens)
    q = to_dev(inp.query)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    graph = _capture(lambda: pa.pa_reshape_and_decode_fp8(out, q, nk, nv, sm, kc, vc, bt, cl, cfg.scale,
                                                          cfg.k_scale, cfg.v_scale, lse_out=lse))

    def eager(qr):
        kce, vce = to_dev(kc0), to_dev(vc0)
        oe, le = torch.empty_like(q), torch.empty_like(lse)
        pa.pa_reshape_and_decode_fp8(oe, qr, nk, nv, sm, kce, vce, bt, cl, cfg.scale, cfg.k_scale, cfg.v_scale,
                                     lse_out=le)
        torch.cuda.synchronize()
        return oe, le, kce, vce

    _replay_against_eager(q, _queries(q.shape, q.dtype, REPLAYS, 5), graph, [out, lse, kc, vc], eager)


@pytest.mark.parametrize("split", [False, True])
def test_multi_query_graph(pa, split):
    base = W.small_case("graph_mq", 10, 32, 8, 128, "bf16", ("uniform", 1, 2), seed=63, num_blocks=400)
    mq = W.make_multi_inputs(W.MultiQueryConfig("graph_mq", base, ("fixed", 1)),
                             context_lens=np.array([600, 5, 90, 17, 300, 1, 640, 33, 200, 48], np.int32),
                             query_lens=np.array([5, 5, 1, 17, 37, 1, 3, 9, 1, 2], np.int32))
    p = mq.paged
    kc, vc, bt = to_dev(p.key_cache), to_dev(p.value_cache), to_dev(p.block_tables)
    cl, loc = to_dev(p.context_lens), to_dev(mq.query_start_loc)
    q = to_dev(mq.query)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    max_ctx = int(p.context_lens.max())
    ws = torch.empty(pa.pa_multi_query_split_workspace_bytes(mq.num_tokens, 32, 128, max_ctx, 128),
                     dtype=torch.uint8, device="cuda")

    def call(o, qq, le, w):
        if split:
            pa.pa_multi_query_split(o, qq, kc, vc, bt, cl, loc, base.scale, max_ctx, 128, w, lse_out=le)
        else:
            pa.pa_multi_query(o, qq, kc, vc, bt, cl, loc, base.scale, lse_out=le)

    graph = _capture(lambda: call(out, q, lse, ws))

    def eager(qr):
        oe, le = torch.empty_like(q), torch.empty_like(lse)
        call(oe, qr, le, torch.empty_like(ws))
        torch.cuda.synchronize()
        return oe, le

    _replay_against_eager(q, _queries(q.shape, q.dtype, REPLAYS, 3), graph, [out, lse], eager)
