"""pa_decode_split_noalloc, whose workspace is the library's own per-GPU
device array (no allocation), against pa_decode_split with a caller
workspace: bit-identical outputs and log-sum-exps, and the oracle's answers,
on two calls in a row with the second one smaller (the array keeps the first
call's contents), for each cut; and the size limit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_TOL, TOL, Dev, bits, ensure_built, forced, max_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return ensure_built()


def _both(pa, d, P):
    """pa_decode_split (caller workspace) and pa_decode_split_noalloc on the same inputs."""
    inp = d.inp
    mcl = inp.max_context_len
    out_ref, lse_ref, _ = d.decode_split(pa, partition_size=P, lse=True)
    out = torch.full_like(d.q, float("nan"))
    lse = torch.full(d.q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_decode_split_noalloc(out, d.q, d.kc, d.vc, d.bt, d.cl, d.cfg.scale, mcl, P, lse_out=lse)
    torch.cuda.synchronize()
    return out_ref, lse_ref, out, lse


@pytest.mark.parametrize("cut", [0, 1, 2], ids=["default", "partitions", "pieces"])
def test_noalloc_equals_split_on_two_calls(pa, cut):
    big = W.make_inputs(W.CONFIG_BY_NAME["long_split"], mode="parity")
    small_cfg = W.small_case("noalloc_small", 5, 16, 4, 128, "bf16", ("uniform", 1, 700), seed=81, num_blocks=300,
                             partition_size=64)
    small = W.make_inputs(small_cfg, mode="parity")
    with forced(pa, split_cut=cut):
        for inp, P in ((big, 512), (small, 64)):
            need = pa.pa_decode_split_workspace_bytes(inp.cfg.num_seqs, inp.cfg.num_heads, inp.cfg.head_size,
                                                      inp.max_context_len, P)
            print(f"[noalloc] {inp.cfg.name} cut {cut}: workspace {need} bytes", flush=True)
            assert need <= pa.PA_DECODE_SPLIT_NOALLOC_MAX_BYTES
            d = Dev(inp)
            out_ref, lse_ref, out, lse = _both(pa, d, P)
            np.testing.assert_array_equal(bits(out), bits(out_ref))
            np.testing.assert_array_equal(bits(lse), bits(lse_ref))
            ref, ref_lse = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                               inp.context_lens, inp.cfg.scale, inp.cfg.dtype)
            assert max_err(out, ref) <= TOL[inp.cfg.dtype]
            assert max_err(lse, ref_lse) <= LSE_TOL[inp.cfg.dtype]


def test_noalloc_rejects_a_workspace_past_its_limit(pa):
    cfg = W.small_case("noalloc_limit", 4, 32, 8, 128, "bf16", ("uniform", 1, 40), seed=82, num_blocks=16)
    d = Dev(W.make_inputs(cfg))
    S, Hq, dh = d.q.shape
    P = 16
    mcl = 1 << 20
    assert pa.pa_decode_split_workspace_bytes(S, Hq, dh, mcl, P) > pa.PA_DECODE_SPLIT_NOALLOC_MAX_BYTES
    out = torch.full_like(d.q, float("nan"))
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_split_noalloc(out, d.q, d.kc, d.vc, d.bt, d.cl, cfg.scale, mcl, P)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool(torch.isnan(out.float()).all())
