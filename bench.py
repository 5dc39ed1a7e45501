#!/usr/bin/env python3
"""Benchmark: paged GQA attention on one MI355X.

Headline workload: long-context decode (batch 1, 32 query / 8 KV heads,
head_dim 128, context 32768, page size 16, shuffled pages in a 4096-page
pool, bf16) with split-KV and the log-sum-exp merge.  One step = one decode
call (every stage of the path) for the whole batch, replayed from a HIP
graph.  Each step reads a different copy of the K/V pools (--pools copies,
together far larger than the 256 MiB Infinity Cache), so every step streams
its KV bytes from HBM.

Reported: decode KV GB/s = 4096 bytes per context token (8 KV heads x K and
V x 128 x 2 bytes) x context tokens / step time.  Alongside, under
"configs", every workload of the five-config set, each timed the same way
(graph replays, inputs rotated over copies that together exceed the
Infinity Cache) with its own roofline: decode lines against 8 TB/s of HBM,
the causal chunked prefill against the dense bf16 MFMA peak (TFLOP/s over
the causally allowed pairs, 4*D flops per (query, key, head)), the mixed
batch against whichever of the two bounds its bytes and flops make larger.
Then the paged append, and the fp64 oracle timed on the host cores.

    python bench.py [--gpus 1] [--steps 60] [--warmup 10]
"""
import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
DECODE_BYTES_PER_TOKEN = 4096

# HBM bytes per call from rocprofv3 FETCH_SIZE + WRITE_SIZE counters (each
# scaled by what it reads for a plain 256 MiB device copy), for the kernels
# and launch shapes as last profiled, on head-major pools (the default
# --layout); None where they changed since.
TRAFFIC = {
    # decode_kernel<4,4,false> + splitkv_reduce_kernel, 32 splits
    # (profiles/decode_ctx32k_hbm_counters.md)
    "decode_ctx32k": 135727556,
    # decode_kernel<4,4,false> + splitkv_reduce_kernel, 8 splits
    # (profiles/decode_ctx512_hbm_counters.md)
    "decode_ctx512": 2691108,
    # decode_even_kernel<4,4> + unit_merge_kernel, split bound 4
    # (profiles/decode_b64_hbm_counters.md)
    "decode_b64": 1141282078,
    # decode_even_kernel<4,8> + unit_merge_kernel, split bound 128
    # (profiles/decode_b256_ctx8k_hbm_counters.md)
    "decode_b256_ctx8k": 8598634829,
}
# The same for one pa_prefill call (unified kernel, + merges when present).
PREFILL_TRAFFIC = {
    # unified_kernel<4,false,128> (profiles/prefill_chunk2048_hbm_counters.md)
    "prefill_chunk2048": 184939303,
    # unified_kernel<4,false,128> + splitkv_reduce_kernel
    # (profiles/mixed_unified_hbm_counters.md)
    "mixed_unified": 643197379,
    # verify_kernel<4,1,false,128> + unit_merge_kernel
    # (profiles/spec_verify_b64_hbm_counters.md)
    "spec_verify_b64": 1203498318,
}

# The same for one pa_cache_append call.
APPEND_TRAFFIC = {
    # append_kernel (profiles/append_prefill_chunk2048_hbm_counters.md)
    "prefill_chunk2048": 67198731,
}


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_ctx32k")
    ap.add_argument("--pools", type=int, default=6, help="K/V pool copies cycled over steps")
    ap.add_argument("--splits", type=int, default=0, help="force num_splits (0 = table)")
    ap.add_argument("--waves", type=int, default=0, help="force waves per workgroup (0 = table)")
    ap.add_argument("--variant", type=int, default=-1, help="force pa_tiles.variant (-1 = table)")
    ap.add_argument("--layout", default="head_major", choices=("head_major", "token_major"),
                    help="storage order of the K/V pools' pages (same values, other strides); "
                         "the run also times the headline workload in the other order")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-workload", default="prefill_chunk2048",
                    help="workload of --prefill-only (prefill_chunk2048 or mixed_unified)")
    ap.add_argument("--append-only", action="store_true",
                    help="time only pa_cache_append on --prefill-workload (for profiling)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill workload (profiling runs)")
    ap.add_argument("--prefill-shape", default="", choices=("",) + tuple(PREFILL_SHAPES),
                    help="--prefill-only at another shape: head dim 64 or 256, or G = 16 "
                         "(64 q / 4 KV heads), same lengths")
    ap.add_argument("--prefill-tile-splits", type=int, default=-1,
                    help="--prefill-only with pa_tiles.tile_splits forced (-1 = table)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after timing, run 4 plain device copies of MIB MiB (a known-size "
                         "kernel for scaling HBM byte counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--launch-study", action="store_true",
                    help="time one decode step eagerly, as one graph replay, and as one of "
                         "eight steps in a replay, per decode workload; print one JSON line")
    ap.add_argument("--all", action="store_true",
                    help="also time the extra workloads (decode_b256_ctx8k, spec_verify_b64, "
                         "the decode_b64 append) and report them under 'others'")
    return ap.parse_args()


def decode_bytes(b):
    return int(b.context_lens.sum().item()) * DECODE_BYTES_PER_TOKEN


def prefill_flops(b):
    """4*D flops per causally allowed (query, key, q-head) triple."""
    D, Hq = b.spec.head_dim, b.spec.num_q_heads
    total = 0
    for L, q in zip(b.context_lens.tolist(), b.query_lens):
        # query i (0-based) of the chunk sees L - q + i + 1 keys
        total += q * (L - q) + q * (q + 1) // 2 if b.spec.causal else q * L
    return 4 * D * Hq * total


def spread(per_ms):
    """p10 / median / p90 of the time per step over the timed steps, in us
    (a step's time is the average over the graph replay that holds it)."""
    xs = sorted(per_ms)
    if not xs:
        return None

    def q(f):
        return round(xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))] * 1e3, 2)

    return {"p10_us": q(0.1), "p50_us": q(0.5), "p90_us": q(0.9), "steps": len(xs)}


def whole_replays(steps, per):
    """Secondary lines time a whole number of multi-step replays: a replay of
    a single step costs 5-10 us more on this stack (see --launch-study)."""
    return -(-steps // per) * per


def time_replays(torch, graph_all, singles, steps, warmup):
    """Time exactly `steps` steps: replays of graph_all (one step per pool
    copy, len(singles) steps each), then single-step graphs for the rest.
    HIP events on the replay stream bracket every replay.  Returns
    (total ms, ms per step of each replay)."""
    per_all = len(singles)
    for i in range(warmup):
        singles[i % per_all].replay()
    torch.cuda.synchronize()
    plan = [(graph_all, per_all)] * (steps // per_all)
    plan += [(singles[i], 1) for i in range(steps % per_all)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i, (g, _) in enumerate(plan):
        g.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = []
    for i, (_, n) in enumerate(plan):
        per += [evs[i].elapsed_time(evs[i + 1]) / n] * n
    return evs[0].elapsed_time(evs[-1]), per


def bench_decode(torch, pa, workloads, args, dev):
    spec = workloads.WORKLOADS[args.workload]
    if not spec.decode_layout:
        raise SystemExit(f"{args.workload} is not a decode workload")
    b = workloads.with_layout(workloads.generate(spec, dev, fill="zero"), args.layout)
    note(f"generated {spec.name}: B={b.num_seqs} max_ctx={b.max_context_len} ({args.layout})")
    pools = [(b.k_pool, b.v_pool)]
    for _ in range(max(1, args.pools) - 1):
        pools.append((b.k_pool.clone(), b.v_pool.clone()))
    max_ctx = b.max_context_len  # host bound, read once outside any capture
    problem = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale, max_ctx, 1)
    tiles, ws = pa.select_tiles(problem)
    if args.splits or args.waves or args.variant >= 0:
        tiles.num_splits = args.splits or tiles.num_splits
        tiles.waves_per_wg = args.waves or tiles.waves_per_wg
        tiles.variant = args.variant if args.variant >= 0 else tiles.variant
        ws = pa.workspace_size(problem, tiles)
    workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)  # counters start at 0
    out = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)

    def step(kp, vp):
        pa.decode(b.q, kp, vp, b.block_tables, b.context_lens, spec.scale, max_ctx,
                  out=out, tiles=tiles, workspace=workspace, problem=problem)

    for kp, vp in pools:  # eager warm-up (and first-launch costs) outside capture
        step(kp, vp)
    torch.cuda.synchronize()
    singles = []
    for kp, vp in pools:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(kp, vp)
        singles.append(g)
    g_all = torch.cuda.CUDAGraph()  # one decode step per pool copy, back to back
    with torch.cuda.graph(g_all):
        for kp, vp in pools:
            step(kp, vp)
    torch.cuda.synchronize()
    note(f"captured decode graphs ({len(pools)} steps per replay), tiles={tiles.as_dict()}")
    total_ms, per = time_replays(torch, g_all, singles, args.steps, args.warmup)
    nbytes = decode_bytes(b)
    return dict(batch=b, tiles=tiles, total_ms=total_ms, per=per, nbytes=nbytes,
                pool_bytes=sum(p[0].numel() * 2 * 2 for p in pools))


def decode_line(torch, pa, workloads, args, dev):
    """A decode workload as a secondary line: time per step, KV GB/s and its
    HBM roofline."""
    args = argparse.Namespace(**{**vars(args), "steps": whole_replays(args.steps, args.pools)})
    dd = bench_decode(torch, pa, workloads, args, dev)
    ms = dd["total_ms"] / args.steps
    gbs = dd["nbytes"] / (ms * 1e-3) / 1e9
    return {"workload": args.workload, "metric": "decode KV GB/s (4096 B per context token)",
            "value": round(gbs, 1), "unit": "GB/s", "us_per_step": round(ms * 1e3, 2),
            "step_us": spread(dd["per"]), "kv_layout": args.layout,
            "bytes_per_step": dd["nbytes"], "pool_copies": args.pools,
            "rotated_mib": round(dd["pool_bytes"] / 2 ** 20, 1),
            "tiles": dd["tiles"].as_dict(),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": TRAFFIC.get(args.workload)}}


def prefill_bytes(b):
    """KV bytes the causal rows read (4096 per key) plus Q and O."""
    kv = 0
    for L, q in zip(b.context_lens.tolist(), b.query_lens):
        kv += L * DECODE_BYTES_PER_TOKEN if q else 0
    qo = 2 * b.q.numel() * 2
    return kv + qo


def roofline(nbytes, flops, ms, traffic):
    """Roofline of one step of `ms` milliseconds: bound by whichever of
    bytes / HBM peak and flops / MFMA peak is the larger; achieved and peak
    in that bound's unit, frac = achieved / peak (for the bound that sets
    the ideal time this is the whole-launch fraction)."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFS * 1e12)
    sec = ms * 1e-3
    if t_hbm >= t_mfma:
        a = nbytes / sec / 1e9
        return {"bound": "hbm", "achieved": round(a, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic}
    a = flops / sec / 1e12
    return {"bound": "mfma", "achieved": round(a, 2), "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s", "frac": round(a / MFMA_BF16_PEAK_TFS, 4), "traffic": traffic}


# Other shapes of a prefill workload (profiling runs): same lengths and seed.
PREFILL_SHAPES = {"d64": dict(head_dim=64), "d256": dict(head_dim=256),
                  "g16": dict(num_q_heads=64, num_kv_heads=4)}


def shaped_workload(workloads, name, shape):
    """Name of workload `name` at `shape` (a PREFILL_SHAPES key; "" = as
    defined), registered in workloads.WORKLOADS on first use."""
    if not shape:
        return name
    shaped = f"{name}_{shape}"
    if shaped not in workloads.WORKLOADS:
        workloads.WORKLOADS[shaped] = dataclasses.replace(
            workloads.WORKLOADS[name], name=shaped, **PREFILL_SHAPES[shape])
    return shaped


def bench_prefill(torch, pa, workloads, dev, steps, warmup, name="prefill_chunk2048",
                  copies=3, layout="head_major", tile_splits=-1):
    """One pa_prefill call per step, four steps per graph replay.  Each step
    reads a different copy of Q and of the pools and writes a different
    output (`copies` of them, together larger than the 256 MiB Infinity
    Cache), so no step finds its inputs in that cache."""
    spec = workloads.WORKLOADS[name]
    b = workloads.with_layout(workloads.generate(spec, dev, fill="zero"), layout)
    max_ctx, max_q = b.max_context_len, b.max_query_len
    problem = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                              max_ctx, max_q, causal=spec.causal)
    tiles, ws = pa.select_tiles(problem)
    if tile_splits >= 0:
        tiles.tile_splits = tile_splits
        ws = pa.workspace_size(problem, tiles)
    workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
    sets = [(b.q, b.k_pool, b.v_pool, torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev))]
    for _ in range(max(1, copies) - 1):
        sets.append((b.q.clone(), b.k_pool.clone(), b.v_pool.clone(),
                     torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)))

    def step(q, kp, vp, out):
        pa.prefill(q, b.query_start_loc, kp, vp, b.block_tables, b.context_lens,
                   spec.scale, max_ctx, max_q, causal=spec.causal,
                   out=out, tiles=tiles, workspace=workspace, problem=problem)

    for st in sets:
        step(*st)
    torch.cuda.synchronize()
    per_replay = 4  # back to back, as a serving loop issues them
    singles = []
    for i in range(per_replay):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(*sets[i % len(sets)])
        singles.append(g)
    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all):
        for i in range(per_replay):
            step(*sets[i % len(sets)])
    total_ms, per = time_replays(torch, g_all, singles, whole_replays(steps, per_replay), warmup)
    flops = prefill_flops(b)
    nbytes = prefill_bytes(b)
    avg_ms = sum(per) / len(per)
    tfs = flops / (avg_ms * 1e-3) / 1e12
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    rl = roofline(nbytes, flops, avg_ms, PREFILL_TRAFFIC.get(name))
    set_bytes = sum(t.numel() * t.element_size() for t in sets[0])
    return {"workload": name,
            "metric": "attention TFLOP/s over causal pairs (4*D flop each) and GB/s of "
                      "K/V + Q + O bytes",
            "value": round(tfs, 2), "unit": "TFLOP/s", "us_per_step": round(avg_ms * 1e3, 2),
            "ms_per_step": round(avg_ms, 4), "step_us": spread(per), "kv_layout": layout,
            "gb_per_s": round(gbs, 1),
            "flops_per_step": flops, "bytes_per_step": nbytes,
            "input_copies": len(sets),
            "rotated_mib": round(len(sets) * set_bytes / 2 ** 20, 1),
            "tiles": tiles.as_dict(), "roofline": rl}


def append_bytes(b):
    """Algorithmic bytes of a paged KV append: each new token's K and V rows
    (Hkv * D bf16 each) read once and written once."""
    return b.num_tokens * b.spec.num_kv_heads * b.spec.head_dim * 2 * 2 * 2


def bench_append(torch, pa, workloads, dev, steps, warmup, name="prefill_chunk2048",
                 copies=8, pool_copies=8, layout="head_major"):
    """pa_cache_append of a batch's new tokens, eight steps per graph replay.
    Each step appends a different copy of the new rows, into a different copy
    of the pools when pool_copies = copies (copies of both together exceed the
    256 MiB Infinity Cache for the chunked prefill), so the rows stream from
    HBM and the written pages leave for HBM."""
    spec = workloads.WORKLOADS[name]
    b = workloads.with_layout(workloads.generate(spec, dev, fill="zero"), layout)
    sets = []
    for i in range(copies):
        kn, vn = workloads.new_kv(b, seed=500 + i)
        if i < pool_copies:
            kp, vp = (b.k_pool, b.v_pool) if i == 0 else (b.k_pool.clone(), b.v_pool.clone())
        sets.append((kn, vn, kp, vp))
    problem = pa.make_problem(sets[0][0], b.k_pool, b.block_tables, b.num_seqs, 1.0, 0, 1)

    def step(kn, vn, kp, vp):
        pa.cache_append(kn, vn, kp, vp, b.block_tables, b.context_lens, b.query_start_loc,
                        problem=problem)

    for st in sets:
        step(*st)
    torch.cuda.synchronize()
    singles = []
    for st in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(*st)
        singles.append(g)
    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all):
        for st in sets:
            step(*st)
    total_ms, per = time_replays(torch, g_all, singles, whole_replays(steps, len(singles)), warmup)
    avg_ms = sum(per) / len(per)
    nbytes = append_bytes(b)
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    return {"workload": f"{name}: append {b.num_tokens} new tokens x {spec.num_kv_heads} kv "
                        f"heads (K and V) into their pages",
            "metric": "paged KV append GB/s (new rows read + written)",
            "value": round(gbs, 1), "unit": "GB/s", "us_per_step": round(avg_ms * 1e3, 2),
            "step_us": spread(per), "kv_layout": layout, "bytes_per_step": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": APPEND_TRAFFIC.get(name)}}


def launch_study(torch, pa, workloads, dev, reps=40):
    """Launch overhead of a decode step on this chip: the same pa_decode call
    issued eagerly from Python (two kernel launches through the C ABI), as a
    one-step graph replay, and inside an eight-step graph replay.  The pools
    are not rotated, so short contexts are served from the caches: this
    isolates launch cost, not bandwidth."""
    out = {}
    for name in ("decode_ctx512", "decode_ctx32k", "decode_b64"):
        spec = workloads.WORKLOADS[name]
        b = workloads.generate(spec, dev, fill="zero")
        max_ctx = b.max_context_len
        pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale, max_ctx, 1)
        tiles, ws = pa.select_tiles(pb)
        workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        o = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)

        def step():
            pa.decode(b.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, spec.scale,
                      max_ctx, out=o, tiles=tiles, workspace=workspace, problem=pb)

        def timed(fn, n_per):
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (reps * n_per)

        eager = timed(step, 1)
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1):
            step()
        g8 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g8):
            for _ in range(8):
                step()
        out[name] = {"eager_us": round(eager, 2), "graph_1_us": round(timed(g1.replay, 1), 2),
                     "graph_8_us": round(timed(g8.replay, 8), 2),
                     "kernels_per_step": 2 if tiles.num_splits > 1 else 1}
        note(f"{name}: {out[name]}")
        del b, g1, g8
        torch.cuda.empty_cache()
    return out


def calibrate_copy(torch, dev, mib):
    """Plain device-to-device copies of a known size (for counter scaling)."""
    if mib <= 0:
        return
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    note(f"calibration: 4 copies of {mib} MiB")


def measured_copy_peak(torch, dev, mib=1024, reps=10):
    """HBM rate of a plain device-to-device copy (torch) of `mib` MiB, bytes
    read + written: the practical streaming rate of this machine, reported as
    context beside the spec peak."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"kind": f"device-to-device copy of {mib} MiB (torch), read + written bytes",
            "gb_per_s": round(gbs, 1), "frac_of_spec": round(gbs / HBM_PEAK_GBS, 4)}


def cpu_baseline(workloads, b, seconds):
    """The fp64 oracle on the same decode workload, on the host cores."""
    import oracle
    import numpy as np
    qsl = None
    inp = oracle.PagedInputs(
        q=workloads.bf16_bits(b.q), k_pool=workloads.bf16_bits(b.k_pool),
        v_pool=workloads.bf16_bits(b.v_pool), block_tables=b.block_tables.cpu().numpy(),
        context_lens=b.context_lens.cpu().numpy(), query_start_loc=qsl,
        num_kv_heads=b.spec.num_kv_heads, page_size=b.spec.page_size,
        strides=b.host_strides(), scale=b.spec.scale, causal=b.spec.causal)
    threads = oracle.default_threads()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(inp, threads=threads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds or runs >= 1000:
            break
    gbs = decode_bytes(b) * runs / el / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"whole {b.spec.name} batch (all {b.q.shape[0] * b.q.shape[1]} query "
                      f"rows), {runs} run(s) in {el:.1f} s, fp64, {threads} threads"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this library is a "
              "single-GPU kernel library.  Attention shards across GPUs by KV head or by "
              "sequence with no communication; very long contexts would shard by page range "
              "and merge the (O, lse) partials with pa_splitkv_reduce after an all-gather.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from paged_gqa_attention_pa_amd import pa, workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pa.load()
    dev = torch.device("cuda:0")

    if args.launch_study:
        print(json.dumps({"launch_study": launch_study(torch, pa, workloads, dev)}), flush=True)
        return
    if args.append_only:
        app = bench_append(torch, pa, workloads, dev, args.steps, args.warmup,
                           name=args.prefill_workload, layout=args.layout)
        note(f"append: {app['us_per_step']} us, {app['value']} GB/s")
        calibrate_copy(torch, dev, args.calibrate_copy)
        print(json.dumps(app), flush=True)
        return
    if args.prefill_only:
        pre = bench_prefill(torch, pa, workloads, dev, args.steps, args.warmup,
                            name=shaped_workload(workloads, args.prefill_workload,
                                                 args.prefill_shape),
                            layout=args.layout, tile_splits=args.prefill_tile_splits)
        note(f"prefill: {pre['value']} TFLOP/s")
        calibrate_copy(torch, dev, args.calibrate_copy)
        print(json.dumps(pre), flush=True)
        return
    d = bench_decode(torch, pa, workloads, args, dev)
    b = d["batch"]
    ms_per_step = d["total_ms"] / args.steps
    value = d["nbytes"] / (ms_per_step * 1e-3) / 1e9
    avg_launch_ms = sum(d["per"]) / len(d["per"])
    achieved = d["nbytes"] / (avg_launch_ms * 1e-3) / 1e9
    note(f"decode: {ms_per_step * 1e3:.2f} us/step, {value:.1f} GB/s")

    result = {
        "metric": "decode KV GB/s (% of HBM peak); prefill attention TFLOP/s (% MFMA peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "step_us": spread(d["per"]),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, Llama-3.1-8B-shaped attention, no weights)",
        "config": {
            "workload": f"{b.spec.name}: decode, batch {b.num_seqs}, context "
                        f"{b.max_context_len}, 32 q / 8 kv heads, head_dim 128, page 16, "
                        f"pool {b.spec.pool_pages} pages",
            "num_splits": d["tiles"].num_splits,
            "waves_per_wg": d["tiles"].waves_per_wg,
            "variant": d["tiles"].variant,
            "pool_copies": args.pools,
            "kv_bytes_per_step": d["nbytes"],
            "graph": "hipGraph replays, one decode step per pool copy in each",
            "kv_layout": args.layout,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": TRAFFIC.get(args.workload),
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
        },
    }
    del d, b
    torch.cuda.empty_cache()
    if not args.no_prefill:
        # the same headline workload with the pools' pages in the other
        # storage order (same values, same kernels and launch shape)
        other = "token_major" if args.layout == "head_major" else "head_major"
        sub = argparse.Namespace(**{**vars(args), "layout": other})
        result["other_layout"] = decode_line(torch, pa, workloads, sub, dev)
        note(f"{args.workload} ({other}): {result['other_layout']['us_per_step']} us, "
             f"{result['other_layout']['value']} GB/s")
        torch.cuda.empty_cache()
        # Every config of the five-config set, each with its own roofline.
        # Pool copies per decode step: enough that the copies cycled exceed
        # the 256 MiB Infinity Cache (64 pages x 2 pools x 32 KiB = 4 MiB per
        # copy at context 512; one decode_b64 step already reads 1.09 GB).
        configs = {}
        for name, pools in (("decode_ctx512", 96), ("decode_ctx32k", args.pools),
                            ("decode_b64", 2)):
            if name == args.workload:
                configs[name] = {"same_as": "headline"}
                continue
            sub = argparse.Namespace(**{**vars(args), "workload": name, "splits": 0, "waves": 0,
                                        "variant": -1, "pools": pools})
            configs[name] = decode_line(torch, pa, workloads, sub, dev)
            note(f"{name}: {configs[name]['us_per_step']} us, {configs[name]['value']} GB/s")
            torch.cuda.empty_cache()
        for name, copies in (("prefill_chunk2048", 3), ("mixed_unified", 2)):
            configs[name] = bench_prefill(torch, pa, workloads, dev, max(8, args.steps // 2),
                                          max(8, args.warmup), name=name, copies=copies,
                                          layout=args.layout)
            c = configs[name]
            note(f"{name}: {c['us_per_step']} us, {c['value']} TFLOP/s, {c['gb_per_s']} GB/s, "
                 f"roofline {c['roofline']['bound']} {c['roofline']['frac']}")
            torch.cuda.empty_cache()
        result["configs"] = configs
        result["append"] = bench_append(torch, pa, workloads, dev, max(16, args.steps // 2),
                                        max(8, args.warmup), layout=args.layout)
        note(f"append: {result['append']['us_per_step']} us, {result['append']['value']} GB/s")
    if args.all:
        others = {}
        sub = argparse.Namespace(**{**vars(args), "workload": "decode_b256_ctx8k", "splits": 0,
                                    "waves": 0, "variant": -1, "pools": 1})
        others["decode_b256_ctx8k"] = decode_line(torch, pa, workloads, sub, dev)
        note(f"decode_b256_ctx8k: {others['decode_b256_ctx8k']}")
        torch.cuda.empty_cache()
        spec_v = bench_prefill(torch, pa, workloads, dev, max(8, args.steps // 2),
                               max(8, args.warmup), name="spec_verify_b64", copies=2,
                               layout=args.layout)
        others["spec_verify_b64"] = spec_v
        note(f"spec_verify_b64: {spec_v['us_per_step']} us, {spec_v['gb_per_s']} GB/s")
        app = bench_append(torch, pa, workloads, dev, max(16, args.steps // 2),
                           max(8, args.warmup), name="decode_b64", pool_copies=1,
                           layout=args.layout)
        others["append_decode_b64"] = app
        note(f"append decode_b64: {app['us_per_step']} us")
        result["others"] = others
    mp = measured_copy_peak(torch, dev)
    result["measured_peak"] = mp
    result["roofline"]["frac_of_measured"] = round(result["roofline"]["achieved"] /
                                                   mp["gb_per_s"], 4)
    note(f"measured copy rate: {mp['gb_per_s']} GB/s")
    if not args.no_cpu_baseline:
        spec = workloads.WORKLOADS[args.workload]
        result["cpu_baseline"] = cpu_baseline(workloads, workloads.generate(spec, dev, "zero"),
                                              args.cpu_seconds)
        note(f"cpu baseline: {result['cpu_baseline']}")
    calibrate_copy(torch, dev, args.calibrate_copy)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
