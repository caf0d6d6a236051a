#!/usr/bin/env python3
"""Benchmark of the paged decode hot path on one MI355X.

A step is one pass of the whole path over one batch: reshape_and_cache writes
each sequence's new-token K/V through slot_mapping, then paged decode reads
every context through the block tables (one-pass kernel, or partition kernel
+ log-sum-exp merge with ``--decode split``). Inputs are synthetic, generated
with the shapes of the Llama-3-8B-like batch-256 workload and copied to HBM
before timing; two copies of the KV pool alternate between steps so no step
finds the previous step's K/V in the caches.

Prints ONE JSON line. ``value`` is the effective KV read bandwidth of the
whole step (bytes of K and V the step must read, over step time).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
DEFAULT_WORKLOAD = "llama3_8b_b256"
# Every device source: a stored counter summary is used only if none of them
# changed since it was taken.
KERNEL_SOURCES = ["paged_kv_cache_150_amd/csrc/" + f for f in
                  ("paged_decode.hip", "multi_query.hip", "cache_ops.hip", "pa_device.h", "pa_tiles.h",
                   "pa_internal.h")]
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, vendor figure


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, decode: str, prefix: str = "paged_decode"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_{decode}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def hold_gpu(stream) -> None:
    """Queue a short spin kernel ahead of the timed region so the host can
    enqueue every timed launch before the GPU reaches them: the timed steps
    then run back to back whatever the Python launch overhead."""
    import torch
    with torch.cuda.stream(stream):
        torch.cuda._sleep(50_000_000)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=DEFAULT_WORKLOAD, help="workload name (see workloads.CONFIGS)")
    ap.add_argument("--decode", choices=["fused", "split", "prefix"], default="fused",
                    help="fused: pa_decode (one pass); split: pa_decode_split (partitions + LSE merge)")
    ap.add_argument("--separate-write", action="store_true",
                    help="fused decode: launch pa_reshape_and_cache and pa_decode separately instead of the "
                         "one-launch pa_reshape_and_decode")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--order", choices=["longest", "natural"], default="longest",
                    help="seq_order schedule hint for pa_decode: longest context first (default) or none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle CPU time")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB 20 times (counter calibration) and exit")
    ap.add_argument("--op", choices=["step", "copy_blocks", "multi_query"], default="step",
                    help="step: reshape + decode (the headline); copy_blocks: pa_copy_blocks on the "
                         "workload's pool (copy-on-write copies), one JSON line of its own")
    ap.add_argument("--pairs", type=int, default=4096, help="copy_blocks: block pairs per launch")
    ap.add_argument("--option", action="append", default=[], metavar="NAME=VALUE",
                    help="force a kernel choice (pa_set_option), e.g. tile_waves=4, split_cut=1, "
                         "split_part_factor=2, tile_columns=32, merge_rows=4; repeatable")
    return ap.parse_args()


def apply_options(pa, opts):
    """--option NAME=VALUE pairs -> pa_set_option; returns them as a dict for the JSON line."""
    forced = {}
    for o in opts:
        name, _, value = o.partition("=")
        pa.pa_set_option(getattr(pa, "PA_OPT_" + name.strip().upper()), int(value))
        forced[name.strip()] = int(value)
    return forced


def bench_copy_blocks(args):
    """pa_copy_blocks on the workload's pool shape: `pairs` random (source,
    destination) block pairs per launch, timed with HIP events."""
    import numpy as np
    import torch
    import paged_kv_cache_150_amd as pa
    import workloads as W
    pa.load_library()
    forced = apply_options(pa, args.option)
    cfg = W.CONFIG_BY_NAME[args.config]
    shape = (cfg.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_size)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    kc = torch.zeros(shape, dtype=tdt, device="cuda")
    vc = torch.zeros(shape, dtype=tdt, device="cuda")
    rng = np.random.default_rng(0)
    maps = []
    for _ in range(2):
        ids = rng.permutation(cfg.num_blocks)
        maps.append(torch.from_numpy(np.stack([ids[:args.pairs], ids[args.pairs:2 * args.pairs]], 1)
                                     .astype(np.int64)).cuda())
    stream = torch.cuda.current_stream()
    copy_p = [pa.prepared(pa.pa_copy_blocks, kc, vc, maps[k], stream=stream) for k in range(2)]
    for i in range(args.warmup):
        copy_p[i & 1]()
    torch.cuda.synchronize()
    # One launch per step: the pass timed at its two ends gives the average
    # launch duration; a second pass with events around each launch is kept
    # as a cross-check (those events cost GPU time of their own).
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_gpu(stream)
    t_begin.record(stream)
    for i in range(args.steps):
        copy_p[i & 1]()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_begin.elapsed_time(t_end) / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    hold_gpu(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        copy_p[i & 1]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms_events = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    block_bytes = cfg.block_size * cfg.num_kv_heads * cfg.head_size * (2 if cfg.dtype == "bf16" else 4)
    moved = 2 * 2 * args.pairs * block_bytes  # K and V, read + write
    gbs = moved / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "pa_copy_blocks HBM GB/s (read + write)", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "pairs": args.pairs, "block_bytes": block_bytes,
                   "options": forced or None},
        "launch_ms_events": round(ms_events, 5),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(cfg.name, f"pairs{args.pairs}", "copy_blocks"),
                     "kernel": "pa::copy_blocks_kernel", "algorithmic_bytes_per_launch": moved,
                     "kernel_source_hash": kernel_source_hash()}}))


def bench_multi_query(args):
    """One multi-query step: reshape_and_cache of every new token, then
    pa_multi_query over the whole batch (prompt chunks, speculative positions
    and one-token decodes together). Two pool copies alternate between steps."""
    import numpy as np
    import torch
    import paged_kv_cache_150_amd as pa
    import workloads as W
    pa.load_library()
    forced = apply_options(pa, args.option)
    name = args.config if args.config in W.MQ_CONFIG_BY_NAME else "llama3_8b_b64_spec4"
    cfg = W.MQ_CONFIG_BY_NAME[name]
    base = cfg.base
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    mq_drawn = W.make_multi_inputs(cfg, mode="perf")
    mq = mq_drawn
    if args.order == "longest":
        # The batch listed longest context first (a serving engine orders its
        # batch freely): the tile slots, and so the dispatch, follow it. The
        # batch as drawn is timed as well (natural_order).
        mq = W.reorder_multi_inputs(mq_drawn, np.argsort(-mq_drawn.paged.context_lens, kind="stable"))
    inp = mq.paged
    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    pools = [(up(inp.key_cache), up(inp.value_cache)) for _ in range(2)]
    stream = torch.cuda.current_stream()
    split = args.decode == "split"
    max_ctx = int(inp.context_lens.max(initial=0))
    P = None
    if split:
        # Every context cut into P-token partitions, then the per-row merge.
        P = (args.partition_size or pa.pa_multi_query_split_partition_size(
            base.num_seqs, mq.num_tokens, base.num_heads, base.num_kv_heads, base.head_size, max_ctx) or 1024)
        ws = torch.empty(pa.pa_multi_query_split_workspace_bytes(mq.num_tokens, base.num_heads, base.head_size,
                                                                 max_ctx, P), dtype=torch.uint8, device=dev)

    def calls(m):
        """The step's two launches on batch m, for either pool copy."""
        q, bt, cl, loc = up(m.query), up(m.paged.block_tables), up(m.paged.context_lens), up(m.query_start_loc)
        new_k, new_v, slots = up(m.new_key), up(m.new_value), up(m.slot_mapping)
        out = torch.empty_like(q)
        reshape = [pa.prepared(pa.pa_reshape_and_cache, new_k, new_v, *pools[k], slots, stream=stream)
                   for k in range(2)]
        if split:
            attend = [pa.prepared(pa.pa_multi_query_split, out, q, *pools[k], bt, cl, loc, base.scale, max_ctx, P,
                                  ws, stream=stream) for k in range(2)]
        else:
            attend = [pa.prepared(pa.pa_multi_query, out, q, *pools[k], bt, cl, loc, base.scale, stream=stream)
                      for k in range(2)]
        return reshape, attend

    reshape_p, attend_p = calls(mq)

    print(f"[bench] warmup {args.warmup}, timed {args.steps} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        reshape_p[i & 1]()
        attend_p[i & 1]()
    torch.cuda.synchronize()
    # Step rate from a pass with events only at its ends; per-launch durations
    # from a second pass with events around each attention launch.
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_gpu(stream)
    t_begin.record(stream)
    for i in range(args.steps):
        reshape_p[i & 1]()
        attend_p[i & 1]()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_begin.elapsed_time(t_end) / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    hold_gpu(stream)
    for i in range(args.steps):
        reshape_p[i & 1]()
        ev[i][0].record(stream)
        attend_p[i & 1]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    att = [a.elapsed_time(b) for a, b in ev]
    att_avg = statistics.fmean(att)
    natural_ms = None
    if mq is not mq_drawn:
        nat_reshape, nat_attend = calls(mq_drawn)
        for i in range(args.warmup):
            nat_reshape[i & 1]()
            nat_attend[i & 1]()
        hold_gpu(stream)
        t_begin.record(stream)
        for i in range(args.steps):
            nat_reshape[i & 1]()
            nat_attend[i & 1]()
        t_end.record(stream)
        torch.cuda.synchronize()
        natural_ms = t_begin.elapsed_time(t_end) / args.steps
    kv_bytes = W.algorithmic_kv_bytes(base, inp.context_lens)
    flops = W.multi_query_flops(mq)
    t_hbm = kv_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    step_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    att_gbs = kv_bytes / (att_avg * 1e-3) / 1e9
    att_tflops = flops / (att_avg * 1e-3) / 1e12
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(att_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(att_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(att_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(att_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof.update({"traffic": stored_traffic(cfg.name, "mq_split" if split else "mq", "paged_multi_query"),
                 "kernel": "paged_multi_query_kernel (context partitions) + merge_mq_parts_kernel" if split
                 else "paged_multi_query_kernel", "algorithmic_bytes_per_launch": kv_bytes,
                 "algorithmic_flops_per_launch": flops, "achieved_tflops": round(att_tflops, 2),
                 "kernel_source_hash": kernel_source_hash()})
    T = mq.num_tokens
    rec = {
        "metric": "multi-query paged attention effective KV GB/s (% of HBM peak), 1 GPU",
        "value": round(step_gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": base.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "description": cfg.description, "num_seqs": base.num_seqs,
                   "new_tokens": T, "num_heads": base.num_heads, "num_kv_heads": base.num_kv_heads,
                   "head_size": base.head_size, "block_size": base.block_size, "num_blocks": base.num_blocks,
                   "mean_context": float(inp.context_lens.mean()),
                   "step": "pa_reshape_and_cache + " + ("pa_multi_query_split" if split else "pa_multi_query"),
                   "partition_size": P if split else None, "options": forced or None,
                   "batch_order": "longest context first" if args.order == "longest" else "as drawn"},
        "pct_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes, "attention_ms_avg": round(att_avg, 5),
        "attention_ms_median": round(statistics.median(att), 5),
        "roofline": roof,
    }
    if natural_ms is not None:
        nat_gbs = kv_bytes / (natural_ms * 1e-3) / 1e9
        rec["natural_order"] = {"ms_per_step": round(natural_ms, 5), "value": round(nat_gbs, 1),
                                "pct_hbm_peak": round(100 * nat_gbs / HBM_PEAK_GBS, 2)}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline_multi(mq, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def cpu_baseline_multi(mq, budget_s: float):
    """The fp64 oracle's multi-query attention, sequence by sequence in batch
    order until ~budget_s: KV bytes of the sequences done over the time."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    base, inp = mq.cfg.base, mq.paged
    loc = mq.query_start_loc
    order = np.argsort(-mq.query_lens, kind="stable")  # prompt chunks first, then decodes
    done, passes, t0 = [], 0, time.perf_counter()
    while True:
        for i in order:
            sl = slice(int(loc[i]), int(loc[i + 1]))
            oracle.paged_multi_query(mq.query[sl], inp.key_cache, inp.value_cache, inp.block_tables[i:i + 1],
                                     inp.context_lens[i:i + 1], np.array([0, loc[i + 1] - loc[i]]), base.scale,
                                     base.dtype)
            done.append(int(i))
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            passes += 1
            continue
        break
    dt = time.perf_counter() - t0
    kv = W.algorithmic_kv_bytes(base, inp.context_lens[done])
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle, {passes} whole passes over the {base.num_seqs} sequences and "
                      f"{len(done) - passes * base.num_seqs} more ({int(mq.query_lens[done].sum())} new tokens) "
                      f"in {dt:.1f} s",
            "tokens_per_s": float(mq.query_lens[done].sum()) / dt}


def copy_calibration(mib: int):
    import torch
    n = mib * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 20}))


def cpu_baseline(cfg, inp, budget_s: float):
    """The fp64 oracle on the host cores over the same batch, repeated to ~budget_s."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    reps, t0 = 0, time.perf_counter()
    while True:
        if cfg.cache_dtype == "fp8":
            oracle.paged_decode_fp8(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                    inp.context_lens, cfg.scale, cfg.k_scale, cfg.v_scale)
        else:
            oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables, inp.context_lens,
                                cfg.scale, cfg.dtype)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / reps
    kv = W.algorithmic_kv_bytes(cfg, inp.context_lens)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle, pa_decode of the full {cfg.num_seqs}-sequence batch "
                      f"({reps} passes, {dt:.2f} s each; decode only, no reshape)",
            "seqs_per_s": cfg.num_seqs / dt, "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this path has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.op == "copy_blocks":
        bench_copy_blocks(args)
        return
    if args.op == "multi_query":
        bench_multi_query(args)
        return

    import paged_kv_cache_150_amd as pa
    import workloads as W

    if not os.path.exists(pa.library_path()):
        from paged_kv_cache_150_amd.build import build_library
        build_library()
    pa.load_library()
    forced = apply_options(pa, args.option)

    cfg = W.CONFIG_BY_NAME[args.config]
    P = args.partition_size or cfg.partition_size
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    inp = W.make_inputs(cfg, mode="perf")
    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    fp8 = cfg.cache_dtype == "fp8"
    if fp8 and args.decode != "fused":
        print("bench.py: FP8 caches have the fused decode only (pa_decode_fp8)", file=sys.stderr)
        sys.exit(2)

    # Two resident copies of the pool (same contents), used on alternate steps.
    pools = [(up(inp.key_cache), up(inp.value_cache)) for _ in range(2)]
    q, bt, cl = up(inp.query), up(inp.block_tables), up(inp.context_lens)
    new_k, new_v, slots = up(inp.new_key), up(inp.new_value), up(inp.slot_mapping)
    out = torch.empty_like(q)
    # The schedule a serving loop would pass: it knows every context length on
    # the host when it builds the block tables.
    longest = up(np.argsort(-inp.context_lens, kind="stable").astype(np.int32))
    order = longest if args.order == "longest" else None
    S, Hq, d = cfg.num_seqs, cfg.num_heads, cfg.head_size
    mcl = inp.max_context_len
    ws = torch.empty(max(256, pa.pa_decode_split_workspace_bytes(S, Hq, d, mcl, P),
                         pa.pa_decode_prefix_workspace_bytes(S, Hq, d)), dtype=torch.uint8, device=dev)
    if args.decode == "prefix" and inp.shared_prefix_blocks == 0:
        print(f"bench.py: {cfg.name} has no shared prefix (--decode prefix needs one)", file=sys.stderr)
        sys.exit(2)
    stream = torch.cuda.current_stream()
    # The plain decode step runs as one launch (pa_reshape_and_decode: the
    # new tokens' write folded into the decode) unless asked otherwise.
    one_launch = args.decode == "fused" and not args.separate_write

    def make_step(kc, vc, tables, slot_map, seq_order):
        """(write, attend) callables of one step on these buffers; the binding's
        checks run once here and the calls repeat the bare library calls."""
        if one_launch:
            def fused():
                if fp8:
                    pa.pa_reshape_and_decode_fp8(out, q, new_k, new_v, slot_map, kc, vc, tables, cl, cfg.scale,
                                                 cfg.k_scale, cfg.v_scale, seq_order=seq_order, stream=stream)
                else:
                    pa.pa_reshape_and_decode(out, q, new_k, new_v, slot_map, kc, vc, tables, cl, cfg.scale,
                                             seq_order=seq_order, stream=stream)
            return (lambda: None), pa.prepared(fused)

        def reshape():
            if fp8:
                pa.pa_reshape_and_cache_fp8(new_k, new_v, kc, vc, slot_map, cfg.k_scale, cfg.v_scale, stream=stream)
            else:
                pa.pa_reshape_and_cache(new_k, new_v, kc, vc, slot_map, stream=stream)

        def decode():
            if fp8:
                pa.pa_decode_fp8(out, q, kc, vc, tables, cl, cfg.scale, cfg.k_scale, cfg.v_scale,
                                 seq_order=seq_order, stream=stream)
            elif args.decode == "fused":
                pa.pa_decode(out, q, kc, vc, tables, cl, cfg.scale, seq_order=seq_order, stream=stream)
            elif args.decode == "prefix":
                pa.pa_decode_prefix(out, q, kc, vc, tables, cl, cfg.scale, inp.shared_prefix_blocks, ws,
                                    seq_order=seq_order, stream=stream)
            else:
                pa.pa_decode_split(out, q, kc, vc, tables, cl, cfg.scale, mcl, P, ws, stream=stream)
        return pa.prepared(reshape), pa.prepared(decode)

    steps = [make_step(*pools[k], bt, slots, order) for k in range(2)]
    print(f"[bench] warmup {args.warmup}, timed {args.steps} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        steps[i & 1][0]()
        steps[i & 1][1]()
    torch.cuda.synchronize()

    # The step rate comes from a pass with events only at its two ends (an
    # event between kernels costs GPU time of its own); the per-launch
    # durations of the attention call (with the write folded in, for the
    # one-launch step) from a second pass with events around each launch, on
    # the stream the kernels run on.
    wall0 = time.perf_counter()
    ms_per_step = timed_pass(steps, args.steps, stream)
    wall = time.perf_counter() - wall0
    out_timed = out.clone()
    dec_ms = per_launch_pass(steps, args.steps, stream)
    dec_avg = statistics.fmean(dec_ms)

    kv_bytes = W.algorithmic_kv_bytes(cfg, inp.context_lens)
    step_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    # The shared-prefix decode must read each distinct slot once: its
    # roofline is priced on the unique bytes.
    roof_bytes = W.unique_kv_bytes(inp) if args.decode == "prefix" else kv_bytes
    if one_launch:
        # The launch also reads the new tokens' K/V (query dtype) and writes
        # them to their slots (cache dtype).
        in_bytes = 2 if cfg.dtype == "bf16" else 4
        roof_bytes += (2 * in_bytes + 2 * cfg.kv_elem_bytes) * int(np.count_nonzero(inp.slot_mapping >= 0)) \
            * cfg.num_kv_heads * d
    # With one launch per step the first pass, timed at its two ends over
    # launches queued back to back on the kernel's stream, gives the kernel's
    # average launch duration directly (any gap between launches counts
    # against the kernel); the per-launch events add a cost of their own and
    # are kept as a cross-check.
    launch_ms = ms_per_step if one_launch else dec_avg
    dec_gbs = roof_bytes / (launch_ms * 1e-3) / 1e9

    # What the memory system delivers, measured beside the decode: a plain
    # streaming read of 1 GiB (two buffers, alternating), and the decode's own
    # loads without its arithmetic over the same pools and tables.
    print("[bench] ceilings", file=sys.stderr, flush=True)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    bufs = [torch.ones(1 << 28, dtype=torch.int32, device=dev) for _ in range(2)]
    reads = [(lambda: None, pa.prepared(pa.pa_stream_read, bufs[k], sink, stream=stream)) for k in range(2)]
    for i in range(10):
        reads[i & 1][1]()
    stream_ms = timed_pass(reads, max(50, args.steps // 2), stream)
    ceiling_gbs = (1 << 30) / (stream_ms * 1e-3) / 1e9
    del bufs
    # The access-pattern ceiling is the one-pass decode's; the split and
    # shared-prefix calls read differently and get none.
    gather_ms = gather_gbs = None
    if args.decode == "fused":
        gathers = [(lambda: None, pa.prepared(pa.pa_stream_kv, *pools[k], bt, cl, sink, seq_order=order,
                                              stream=stream)) for k in range(2)]
        for i in range(10):
            gathers[i & 1][1]()
        gather_ms = timed_pass(gathers, args.steps, stream)
        gather_gbs = kv_bytes / (gather_ms * 1e-3) / 1e9

    # The same step in natural sequence order (no seq_order hint), and with
    # every sequence's blocks laid end to end in the pool (contiguous
    # placement, the same contents): the cost of the schedule hint's absence
    # and of scattered placement.
    extra = {}
    if args.decode in ("fused", "prefix") and order is not None:
        nat = [make_step(*pools[k], bt, slots, None) for k in range(2)]
        for i in range(args.warmup):
            nat[i & 1][0]()
            nat[i & 1][1]()
        nat_ms = timed_pass(nat, args.steps, stream)
        extra["natural_order"] = {"ms_per_step": round(nat_ms, 5),
                                  "value": round(kv_bytes / (nat_ms * 1e-3) / 1e9, 1),
                                  "pct_hbm_peak": round(100 * kv_bytes / (nat_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
    ref_ids, tables_c, slots_c = W.contiguous_placement(inp)
    ids_t = up(ref_ids)
    cpools = [(pools[k][0].index_select(0, ids_t), pools[k][1].index_select(0, ids_t)) for k in range(2)]
    bt_c, slots_c_t = up(tables_c), up(slots_c)
    cont = [make_step(*cpools[k], bt_c, slots_c_t, order) for k in range(2)]
    for i in range(args.warmup):
        cont[i & 1][0]()
        cont[i & 1][1]()
    cont_ms = timed_pass(cont, args.steps, stream)
    del cpools
    extra["placement"] = {"shuffled_ms_per_step": round(ms_per_step, 5), "contiguous_ms_per_step": round(cont_ms, 5),
                          "shuffled_over_contiguous": round(ms_per_step / cont_ms, 4),
                          "contiguous_blocks": int(ref_ids.size)}

    # Parity of the timed step's output (the first pass's last step) against
    # the oracle on the same inputs, computed after all timing.
    print("[bench] parity of the timed output against the oracle", file=sys.stderr, flush=True)
    import oracle
    if fp8:
        kc_ref, vc_ref = oracle.reshape_and_cache_fp8(inp.new_key, inp.new_value, inp.key_cache, inp.value_cache,
                                                      inp.slot_mapping, cfg.k_scale, cfg.v_scale)
        ref, _ = oracle.paged_decode_fp8(inp.query, kc_ref, vc_ref, inp.block_tables, inp.context_lens, cfg.scale,
                                         cfg.k_scale, cfg.v_scale)
        del kc_ref, vc_ref
    else:
        ref, _ = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables, inp.context_lens,
                                     cfg.scale, cfg.dtype)
    parity_err = float(np.abs(out_timed.float().cpu().numpy().astype(np.float64) - ref).max())
    tol = 2e-2 if cfg.dtype == "bf16" else 1e-5

    traffic = stored_traffic(cfg.name, args.decode + ("_separate" if args.separate_write else ""))
    one = "paged_multi_query_kernel (one token per sequence)"
    if one_launch:
        one += " with the new-token write"
    split_label = "paged_decode_split_kernel + merge_pieces_kernel"
    if args.decode == "split" and pa.pa_decode_split_part_tokens(
            S, Hq, cfg.num_kv_heads, inp.max_context_len, P,
            pa.PA_DTYPE_BF16 if cfg.dtype == "bf16" else pa.PA_DTYPE_F32):
        split_label = "paged_multi_query_kernel (context partitions) + merge_parts_kernel"
    kernel_label = {"fused": one, "split": split_label,
                    "prefix": "paged_multi_query_kernel (shared prefix) + " + one}[args.decode]
    pct = lambda v: round(float(np.percentile(dec_ms, v)), 5)  # noqa: E731
    rec = {
        "metric": "paged decode attention effective KV GB/s (% of HBM peak) + seqs/sec, 1 GPU",
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "description": cfg.description, "num_seqs": S, "num_heads": Hq,
                   "num_kv_heads": cfg.num_kv_heads, "head_size": d, "block_size": cfg.block_size,
                   "num_blocks": cfg.num_blocks, "mean_context": float(inp.context_lens.mean()),
                   "decode": args.decode, "partition_size": P if args.decode == "split" else None,
                   "seq_order": args.order if args.decode in ("fused", "prefix") else None,
                   "prefix_blocks": inp.shared_prefix_blocks if args.decode == "prefix" else None,
                   "kv_cache": cfg.cache_dtype, "options": forced or None,
                   "step": ("pa_reshape_and_decode_fp8 (one launch)" if fp8 and one_launch else
                            "pa_reshape_and_cache_fp8 + pa_decode_fp8" if fp8 else
                            "pa_reshape_and_decode (one launch)" if one_launch else
                            "pa_reshape_and_cache + " + {"fused": "pa_decode", "split": "pa_decode_split",
                                                         "prefix": "pa_decode_prefix"}[args.decode])},
        "pct_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(S / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "decode_ms_avg": round(dec_avg, 5),
        "decode_ms_median": round(statistics.median(dec_ms), 5),
        "decode_ms_p10": pct(10),
        "decode_ms_p90": pct(90),
        "launch_ms": round(launch_ms, 5),
        "launch_timing": ("timed region / steps (one launch per step)" if one_launch
                          else "HIP events around each launch"),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": kernel_label,
                     "algorithmic_bytes_per_launch": roof_bytes,
                     "measured_ceiling_gbs": round(ceiling_gbs, 1),
                     "measured_ceiling": "pa_stream_read: 1 GiB read once, contiguous range per workgroup, "
                                         "non-temporal 16-byte loads",
                     "frac_of_measured_ceiling": round(dec_gbs / ceiling_gbs, 4),
                     "access_pattern_ceiling_gbs": None if gather_gbs is None else round(gather_gbs, 1),
                     "access_pattern_ceiling": "pa_stream_kv: the one-pass decode's K/V loads over the same "
                                               "pools and tables, no arithmetic (GB/s of algorithmic KV bytes)",
                     "decode_time_over_access_pattern_time": None if gather_ms is None
                     else round(launch_ms / gather_ms, 4),
                     "kernel_source_hash": kernel_source_hash()},
        "parity_max_abs_err": parity_err,
        "parity_tolerance": tol,
        "parity_ok": bool(parity_err <= tol),
        "wall_s_timed": round(wall, 4),  # includes the spin kernel queued ahead of the timed steps
    }
    rec.update(extra)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def timed_pass(steps, n, stream) -> float:
    """Average ms per step of n steps (write then attend, alternating between
    the two entries of `steps`) queued back to back behind a spin kernel, with
    events only at the two ends."""
    import torch
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold_gpu(stream)
    t0.record(stream)
    for i in range(n):
        steps[i & 1][0]()
        steps[i & 1][1]()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


def per_launch_pass(steps, n, stream) -> list:
    """ms of each attention launch of n steps, from events around it."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    hold_gpu(stream)
    for i in range(n):
        steps[i & 1][0]()
        ev[i][0].record(stream)
        steps[i & 1][1]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]

if __name__ == "__main__":
    main()
