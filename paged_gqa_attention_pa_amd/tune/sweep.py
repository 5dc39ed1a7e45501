"""Offline launch-shape sweep on one gfx950 GPU -> the compiled-in tile table.

The runtime never tunes: pa_select_tiles looks shapes up in a table compiled
into the library (the offline micro-benchmark + decision-table idea of the
IBM Triton summary, section on moving autotuning offline, re-derived for this
chip).  This script produces that table:

  python -m paged_gqa_attention_pa_amd.tune.sweep --out-json tune/sweep_gfx950.json
  python -m paged_gqa_attention_pa_amd.tune.sweep --emit-only   # JSON -> header

Decode: for every (units = num_seqs * num_kv_heads, max context) bucket it
times each candidate (num_splits, waves per workgroup, grid variant) on two
length mixes, all contexts equal to the bound and contexts drawn uniformly in
[bound/16, bound], and keeps the candidate with the least summed time relative
to each mix's best.  Prefill: for query-tile workgroup counts and context
bounds it times tile_splits in {1, 2, 4, 8} on prefill-only batches.  Short
query runs (speculative-decode verification, and decode at G = 32 or head dims
other than 128, which run on the same kernel): for (units, context bound)
buckets it times the split bound on several (G, head dim, tokens) shapes and
keeps the one with the least worst relative time over shapes and mixes.

Timing: CUDA graphs of one call per K/V pool copy (copies rotate so the
256 MiB Infinity Cache does not serve the pools), HIP events around replays,
median of the replays.  Inputs are seeded synthetic bf16 N(0,1); Llama-3.1-8B
attention shape (32 query heads, 8 KV heads, head_dim 128, page 16).
"""
import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
GEN_HEADER = os.path.join(PKG, "csrc", "pa_tile_table_gen.h")
DEFAULT_JSON = os.path.join(HERE, "sweep_gfx950.json")

UNIT_BUCKETS = [8, 16, 32, 64, 128, 256, 512, 1024, 2048]      # num_seqs * num_kv_heads
CTX_BUCKETS = [256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072]
MAX_TOKENS = 1 << 21   # batch * context bound per swept shape (8 GiB of K+V)
SPLITS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
WAVES = [4, 8]
VARIANTS = [2, 6]      # static grid + separate merge, even-work grid + separate merge
PF_WG_BUCKETS = [16, 32, 64, 128, 256, 512, 1024]  # query-tile workgroups (tiles x Hkv)
PF_CTX_BUCKETS = [1024, 4096, 16384, 65536]
PF_TILE_SPLITS = [1, 2, 4, 8]
# Short query runs (one Q-block per (sequence, kv head) unit on the even-work
# grid): (G, head dim, query tokens) shapes swept for the split bound.
SHORT_SHAPES = [(4, 128, 4), (8, 128, 4), (4, 64, 1), (4, 256, 1), (32, 128, 1)]
SHORT_SPLITS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
SHORT_UNIT_BUCKETS = [1, 8, 64, 512]
SHORT_CTX_BUCKETS = [1024, 4096, 16384, 32768, 131072]


def log(msg):
    print(msg, flush=True)


def _batch(workloads, name, contexts, queries, seed, dev, slack=2.5):
    # the pool holds `slack` times the pages in use, and each table draws
    # from all of it, as in a serving cache that is partly full
    used = sum(-(-c // 16) for c in contexts)
    spec = workloads.WorkloadSpec(name=name, seed=seed, pool_pages=int(used * slack) + 8,
                                  fixed=list(zip(contexts, queries)),
                                  decode_layout=all(q == 1 for q in queries),
                                  max_blocks=max(1, -(-max(contexts) // 16)))
    return spec, workloads.generate(spec, dev, fill="zero")


def _time_graph(torch, fns, reps=12, warmup=3):
    """Median per-call microseconds of a graph that runs every fn once."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    t = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3 / len(fns))
    del g
    t.sort()
    return t[len(t) // 2]


def sweep_decode(torch, pa, workloads, dev, results):
    for units in UNIT_BUCKETS:
        B = units // 8
        for ctx in CTX_BUCKETS:
            if B * ctx > MAX_TOKENS:
                continue
            key = f"{units}x{ctx}"
            if key in results["decode"]:
                continue
            ntiles = -(-ctx // 16)
            mixes = {"equal": [ctx] * B}
            g = torch.Generator().manual_seed(units * 131 + ctx)
            lo = max(1, ctx // 16)
            mixes["varied"] = torch.randint(lo, ctx + 1, (B,), generator=g).tolist()
            mixes["varied"][0] = ctx  # the bound is reached
            times = {}
            for mix, contexts in mixes.items():
                spec, b = _batch(workloads, f"sw_{key}_{mix}", contexts, [1] * B, 7, dev)
                copies = 2 if B * ctx * 4096 * 2 < (4 << 30) else 1
                pools = [(b.k_pool, b.v_pool)] + [(b.k_pool.clone(), b.v_pool.clone())
                                                 for _ in range(copies - 1)]
                pb = pa.make_problem(b.q, b.k_pool, b.block_tables, B, spec.scale, ctx, 1)
                out = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)
                for S in SPLITS:
                    if S > 1 and S > max(1, ntiles // 4):
                        continue
                    for W in WAVES:
                        for V in VARIANTS:
                            if S == 1 and V == 6:
                                continue
                            t = pa.Tiles(16, S, W, 1, V if S > 1 else 0)
                            ws = torch.zeros(max(pa.workspace_size(pb, t), 256),
                                             dtype=torch.uint8, device=dev)
                            fns = [(lambda kp=kp, vp=vp, t=t, ws=ws: pa.decode(
                                b.q, kp, vp, b.block_tables, b.context_lens, spec.scale, ctx,
                                out=out, tiles=t, workspace=ws, problem=pb))
                                for kp, vp in pools]
                            us = _time_graph(torch, fns)
                            times.setdefault(f"{S},{W},{V if S > 1 else 0}", {})[mix] = round(us, 2)
                del b, pools
                torch.cuda.empty_cache()
            results["decode"][key] = times
            best = min(times.items(), key=lambda kv: sum(kv[1].values()))
            log(f"decode units={units} ctx={ctx}: {len(times)} candidates, best {best}")


def sweep_prefill(torch, pa, workloads, dev, results):
    for wgs in PF_WG_BUCKETS:
        tiles = max(1, wgs // 8)           # query tiles of 64 tokens (G = 4), Hkv = 8
        for ctx in PF_CTX_BUCKETS:
            key = f"{wgs}x{ctx}"
            if key in results["prefill"]:
                continue
            q = min(ctx, 2048)
            B = max(1, -(-tiles * 64 // q))
            if B * ctx > MAX_TOKENS:
                continue
            qlen = min(q, tiles * 64 // B) or 64
            spec, b = _batch(workloads, f"swp_{key}", [ctx] * B, [qlen] * B, 9, dev)
            pb = pa.make_problem(b.q, b.k_pool, b.block_tables, B, spec.scale, ctx, qlen)
            out = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)
            times = {}
            for ts in PF_TILE_SPLITS:
                t, _ = pa.select_tiles(pb)
                t.tile_splits = ts
                ws = torch.zeros(max(pa.workspace_size(pb, t), 256), dtype=torch.uint8,
                                 device=dev)
                fn = (lambda t=t, ws=ws: pa.prefill(
                    b.q, b.query_start_loc, b.k_pool, b.v_pool, b.block_tables, b.context_lens,
                    spec.scale, ctx, qlen, out=out, tiles=t, workspace=ws, problem=pb))
                times[str(ts)] = round(_time_graph(torch, [fn, fn]), 2)
            results["prefill"][key] = times
            log(f"prefill wgs={wgs} ctx={ctx} (B={B} q={qlen}): {times}")
            del b
            torch.cuda.empty_cache()


def _short_batch(workloads, name, contexts, q, G, D, seed, dev, slack=2.5):
    hkv = 1 if G == 32 else 8
    used = sum(-(-c // 16) for c in contexts)
    spec = workloads.WorkloadSpec(name=name, seed=seed, pool_pages=int(used * slack) + 8,
                                  fixed=[(c, q) for c in contexts], num_q_heads=G * hkv,
                                  num_kv_heads=hkv, head_dim=D, decode_layout=(q == 1),
                                  max_blocks=max(1, -(-max(contexts) // 16)))
    return spec, workloads.generate(spec, dev, fill="zero")


def sweep_short(torch, pa, workloads, dev, results):
    res = results.setdefault("short", {})
    for G, D, q in SHORT_SHAPES:
        shape = f"g{G}_d{D}_q{q}"
        per_shape = res.setdefault(shape, {})
        hkv = 1 if G == 32 else 8
        for units in SHORT_UNIT_BUCKETS:
            if units < hkv:
                continue
            B = units // hkv
            for ctx in SHORT_CTX_BUCKETS:
                if B * ctx * hkv * D > MAX_TOKENS * 8 * 128:
                    continue
                key = f"{units}x{ctx}"
                if key in per_shape:
                    continue
                g = torch.Generator().manual_seed(units * 137 + ctx + G + D + q)
                mixes = {"equal": [ctx] * B}
                varied = torch.randint(max(q, ctx // 16), ctx + 1, (B,), generator=g).tolist()
                varied[0] = ctx
                mixes["varied"] = varied
                times = {}
                for mix, contexts in mixes.items():
                    spec, b = _short_batch(workloads, f"sws_{shape}_{key}_{mix}", contexts, q, G,
                                           D, 11, dev)
                    pools = [(b.k_pool, b.v_pool), (b.k_pool.clone(), b.v_pool.clone())]
                    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, B, spec.scale, ctx, q)
                    out = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)
                    for S in SHORT_SPLITS:
                        if S > 1 and S > max(1, -(-ctx // 16) // 4):
                            continue
                        t, _ = pa.select_tiles(pb)
                        t.num_splits = S
                        ws = torch.zeros(max(pa.workspace_size(pb, t), 256), dtype=torch.uint8,
                                         device=dev)
                        if q == 1:
                            fns = [(lambda kp=kp, vp=vp, t=t, ws=ws: pa.decode(
                                b.q, kp, vp, b.block_tables, b.context_lens, spec.scale, ctx,
                                out=out, tiles=t, workspace=ws, problem=pb)) for kp, vp in pools]
                        else:
                            fns = [(lambda kp=kp, vp=vp, t=t, ws=ws: pa.prefill(
                                b.q, b.query_start_loc, kp, vp, b.block_tables, b.context_lens,
                                spec.scale, ctx, q, out=out, tiles=t, workspace=ws, problem=pb))
                                for kp, vp in pools]
                        times.setdefault(str(S), {})[mix] = round(_time_graph(torch, fns), 2)
                    del b, pools
                    torch.cuda.empty_cache()
                per_shape[key] = times
                best = min(times.items(), key=lambda kv: sum(kv[1].values()))
                log(f"short {shape} units={units} ctx={ctx}: best S={best[0]} {best[1]}")


NEAR_TIE = 1.02  # a candidate must beat the default by more than 2% to replace it


def choose(results):
    """Measurements -> per-bucket choices.  A candidate's score is its worse
    time relative to each mix's best; the default launch shape (4 waves,
    even-work grid for batches, static grid for one sequence, at the best
    split count for that shape) is kept unless some candidate scores more
    than 2% better, so noise between near-equal shapes cannot flip the table."""
    dec = {}
    for key, times in results["decode"].items():
        units = int(key.split("x")[0])
        best_mix = {}
        for cand, per in times.items():
            for mix, us in per.items():
                best_mix[mix] = min(best_mix.get(mix, 1e30), us)
        score = {c: max(per[m] / best_mix[m] for m in per) for c, per in times.items()
                 if len(per) == len(best_mix)}
        c = min(score, key=score.get)
        dflt_variant = 6 if units > 8 else 2
        dflt = [d for d in score if d.split(",")[1] == "4" and
                int(d.split(",")[2]) in (dflt_variant, 0)]
        if dflt:
            d = min(dflt, key=score.get)
            if score[d] <= score[c] * NEAR_TIE:
                c = d
        dec[key] = [int(x) for x in c.split(",")]
    pf = {}
    for key, times in results["prefill"].items():
        pf[key] = int(min(times, key=times.get))
    return dec, pf


def choose_short(results):
    """Per (units, context) bucket: the split bound whose worst time relative
    to the best, over every swept short-run shape and both mixes, is least
    (the smaller bound wins a near tie: fewer partials to merge)."""
    rel = {}
    for shape, buckets in results.get("short", {}).items():
        for key, times in buckets.items():
            best = {}
            for S, per in times.items():
                for mix, us in per.items():
                    best[mix] = min(best.get(mix, 1e30), us)
            for S, per in times.items():
                r = max(per[m] / best[m] for m in per)
                cur = rel.setdefault(key, {})
                cur[S] = max(cur.get(S, 0.0), r)
    out = {}
    for key, scores in rel.items():
        ordered = sorted(scores, key=lambda S: int(S))
        c = min(ordered, key=scores.get)
        for S in ordered:  # smallest bound within the tie margin
            if scores[S] <= scores[c] * NEAR_TIE:
                c = S
                break
        out[key] = int(c)
    return out


def emit_header(results, path=GEN_HEADER):
    dec, pf = choose(results)

    def nearest(table, keys_a, keys_b, a, b):
        # fill holes (shapes over the token cap) from the nearest swept context
        if f"{a}x{b}" in table:
            return table[f"{a}x{b}"]
        cands = [kb for kb in keys_b if f"{a}x{kb}" in table]
        if not cands:
            return None
        kb = min(cands, key=lambda x: abs(x - b))
        return table[f"{a}x{kb}"]

    lines = [
        "// Generated by paged_gqa_attention_pa_amd/tune/sweep.py from the gfx950",
        "// measurements in tune/sweep_gfx950.json; regenerate, do not edit.",
        "// Decode: per (units = num_seqs * num_kv_heads, context-bound) bucket the",
        "// (num_splits, waves per workgroup, variant) with the least summed time",
        "// relative to the best on equal and on mixed context lengths.  Prefill:",
        "// tile_splits per (query-tile workgroups, context-bound) bucket.",
        "#pragma once",
        "",
        "namespace pa {",
        "namespace gen {",
        "",
        f"constexpr int kUnitBuckets[] = {{{', '.join(map(str, UNIT_BUCKETS))}}};",
        f"constexpr int kCtxBuckets[] = {{{', '.join(map(str, CTX_BUCKETS))}}};",
        "// {num_splits, waves, variant}; num_splits 0 marks a shape not swept",
        f"constexpr unsigned short kDecode[{len(UNIT_BUCKETS)}][{len(CTX_BUCKETS)}][3] = {{",
    ]
    for u in UNIT_BUCKETS:
        row = []
        for c in CTX_BUCKETS:
            v = nearest(dec, UNIT_BUCKETS, CTX_BUCKETS, u, c) if f"{u}x{c}" in dec else None
            row.append("{%d, %d, %d}" % tuple(v) if v else "{0, 0, 0}")
        lines.append("    {" + ", ".join(row) + "},")
    lines += [
        "};",
        "",
        f"constexpr int kPfWgBuckets[] = {{{', '.join(map(str, PF_WG_BUCKETS))}}};",
        f"constexpr int kPfCtxBuckets[] = {{{', '.join(map(str, PF_CTX_BUCKETS))}}};",
        "// tile_splits; 0 marks a shape not swept",
        f"constexpr unsigned char kPrefillTileSplits[{len(PF_WG_BUCKETS)}][{len(PF_CTX_BUCKETS)}] = {{",
    ]
    for w in PF_WG_BUCKETS:
        row = [str(pf.get(f"{w}x{c}", 0)) for c in PF_CTX_BUCKETS]
        lines.append("    {" + ", ".join(row) + "},")
    short = choose_short(results)
    lines += [
        "};",
        "",
        "// Short query runs: split bound per (units, context-bound) bucket, swept",
        "// over (G, head dim, tokens) = " + ", ".join(f"({g}, {d}, {q})" for g, d, q in SHORT_SHAPES)
        + ";",
        "// 0 marks a shape not swept.",
        f"constexpr int kShortUnitBuckets[] = {{{', '.join(map(str, SHORT_UNIT_BUCKETS))}}};",
        f"constexpr int kShortCtxBuckets[] = {{{', '.join(map(str, SHORT_CTX_BUCKETS))}}};",
        f"constexpr unsigned short kShortSplits[{len(SHORT_UNIT_BUCKETS)}][{len(SHORT_CTX_BUCKETS)}] = {{",
    ]
    for u in SHORT_UNIT_BUCKETS:
        row = [str(short.get(f"{u}x{c}", 0)) for c in SHORT_CTX_BUCKETS]
        lines.append("    {" + ", ".join(row) + "},")
    lines += ["};", "", "}  // namespace gen", "}  // namespace pa", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))
    log(f"wrote {path}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out-json", default=DEFAULT_JSON)
    ap.add_argument("--emit-only", action="store_true", help="regenerate the header from JSON")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-short", action="store_true")
    args = ap.parse_args()
    results = {"decode": {}, "prefill": {}}
    if os.path.exists(args.out_json):
        with open(args.out_json) as f:
            results = json.load(f)
    if not args.emit_only:
        sys.path.insert(0, os.path.dirname(PKG))
        import torch
        from paged_gqa_attention_pa_amd import pa, workloads
        if not torch.cuda.is_available():
            raise SystemExit("the sweep needs a GPU")
        dev = torch.device("cuda:0")
        pa.load()
        results["device"] = torch.cuda.get_device_name(0)
        t0 = time.time()
        try:
            if not args.no_decode:
                sweep_decode(torch, pa, workloads, dev, results)
            if not args.no_prefill:
                sweep_prefill(torch, pa, workloads, dev, results)
            if not args.no_short:
                sweep_short(torch, pa, workloads, dev, results)
        finally:
            with open(args.out_json, "w") as f:
                json.dump(results, f, indent=0, sort_keys=True)
            log(f"sweep {time.time() - t0:.0f} s, results in {args.out_json}")
    emit_header(results)


if __name__ == "__main__":
    main()
