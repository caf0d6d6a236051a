"""The measurement kernels (include/pa_measure.h) run through the C ABI on the
workloads' buffers, leave the sink alone (their checksums never hit the
sentinel on these inputs) and change nothing they read."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import ensure_built, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


@pytest.mark.parametrize("name", ["tiny_f32", "llama3_8b_b64", "llama3_8b_b256_fp8"])
def test_stream_kv_reads_without_writing(pa, name):
    cfg = W.CONFIG_BY_NAME[name]
    inp = W.make_inputs(cfg, mode="perf")
    up = (lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()) if cfg.cache_dtype == "fp8" else to_dev
    kc, vc = up(inp.key_cache), up(inp.value_cache)
    k0, v0 = kc.clone(), vc.clone()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    order = to_dev(np.argsort(-inp.context_lens, kind="stable").astype(np.int32))
    for so in (None, order):
        pa.pa_stream_kv(kc, vc, to_dev(inp.block_tables), to_dev(inp.context_lens), sink, seq_order=so)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    assert torch.equal(kc, k0) and torch.equal(vc, v0)


def test_stream_read(pa):
    src = torch.arange(1 << 22, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    pa.pa_stream_read(src, sink)
    pa.pa_stream_read(src[:1000], sink)          # a short ragged tail (4,000 bytes)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
