"""Offline launch-shape sweep on one gfx950 GPU -> the compiled-in tile table.

The runtime never tunes: pa_select_tiles looks shapes up in a table compiled
into the library (the offline micro-benchmark + decision-table idea of the
IBM Triton summary, section on moving autotuning offline, which also says the
table must be rebuilt per GPU and, by the same token, per shape).  This
script produces that table:

  python -m paged_gqa_attention_pa_amd.tune.sweep --part decode --groups 4
  python -m paged_gqa_attention_pa_amd.tune.sweep --part short
  python -m paged_gqa_attention_pa_amd.tune.sweep --part prefill
  python -m paged_gqa_attention_pa_amd.tune.sweep --emit-only   # JSON -> header

Decode (the decode kernels: head dim 128, G = 1, 2, 4, 8, 16): for every
(units = num_seqs * num_kv_heads, max context) bucket and every G it times
each candidate (num_splits, waves per workgroup, grid variant) on two length
mixes, all contexts equal to the bound and contexts drawn uniformly in
[bound/16, bound].  Short query runs (the short-run kernel: speculative
verification, decode at G = 32 or at head dims 64 and 256): the split bound
per (units, context) bucket for each (head dim, narrow or wide G) key, over
two (G, tokens) shapes of that key.  Prefill: tile_splits per (query-tile
workgroups, context bound) bucket for each head dim.

Choice per bucket: a candidate's score is its worse time relative to each
mix's (and shape's) best.  Candidates within 2% of the best score are ties
(the box-to-box noise); among them the default launch shape (4 waves,
even-work grid for batches) is preferred, then the smallest split count not
below the previous, shorter-context bucket's of the same row, so that rows
grow monotonically with the context unless a measurement says otherwise.

Timing: a CUDA graph of one call per K/V pool copy, with enough copies that
one replay moves at least 512 MiB of K/V (twice the 256 MiB Infinity Cache),
HIP events around the replays, median of the replays.  Inputs are seeded
synthetic bf16 N(0,1), 8 KV heads (1 for the wide-G short-run shapes), page
size 16.
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

DECODE_GROUPS = [1, 2, 4, 8, 16]     # decode kernels, head dim 128, 8 KV heads
UNIT_BUCKETS = [8, 16, 32, 64, 128, 256, 512, 1024, 2048]      # num_seqs * num_kv_heads
CTX_BUCKETS = [256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072]
MAX_TOKENS = 1 << 21   # batch * context bound per swept shape (8 GiB of K+V)
SPLITS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
WAVES = [4, 8]
VARIANTS = [2, 6]      # static grid + separate merge, even-work grid + separate merge
ROTATE_BYTES = 512 << 20  # K/V bytes one timed replay moves at least
MAX_COPIES = 64
PF_DIMS = [64, 128, 256]
PF_WG_BUCKETS = [16, 32, 64, 128, 256, 512, 1024]  # query-tile workgroups (tiles x Hkv)
PF_CTX_BUCKETS = [1024, 4096, 16384, 65536]
PF_TILE_SPLITS = [1, 2, 4, 8]
# Short query runs: keys (head dim, wide = G >= 16) and the (G, tokens)
# shapes timed for each; wide shapes have one KV head.
SHORT_KEYS = [(64, 0), (128, 0), (256, 0), (64, 1), (128, 1), (256, 1)]
SHORT_SHAPES = {0: {64: [(4, 1), (4, 4)], 128: [(4, 4), (8, 2)], 256: [(4, 1), (4, 4)]},
                1: {64: [(32, 1), (16, 2)], 128: [(32, 1), (16, 2)], 256: [(32, 1), (16, 2)]}}
SHORT_SPLITS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
SHORT_UNIT_BUCKETS = [1, 8, 64, 512]
SHORT_CTX_BUCKETS = [1024, 4096, 16384, 32768, 131072]
NEAR_TIE = 1.02  # candidates within 2% of the best score are ties


def log(msg):
    print(msg, flush=True)


def _spec(workloads, name, contexts, queries, seed, G=4, hkv=8, D=128, slack=2.5):
    # the pool holds `slack` times the pages in use, and each table draws
    # from all of it, as in a serving cache that is partly full
    used = sum(-(-c // 16) for c in contexts)
    return workloads.WorkloadSpec(name=name, seed=seed, pool_pages=int(used * slack) + 8,
                                  fixed=list(zip(contexts, queries)), num_q_heads=G * hkv,
                                  num_kv_heads=hkv, head_dim=D,
                                  decode_layout=all(q == 1 for q in queries),
                                  max_blocks=max(1, -(-max(contexts) // 16)))


def _copies(kv_bytes_per_call):
    return max(1, min(MAX_COPIES, -(-ROTATE_BYTES // max(1, kv_bytes_per_call))))


def _pools(b, n):
    return [(b.k_pool, b.v_pool)] + [(b.k_pool.clone(), b.v_pool.clone()) for _ in range(n - 1)]


def _time_graph(torch, fns, reps=9, warmup=2):
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


def _mixes(torch, B, ctx, seed, lo_min=1):
    """Equal lengths, and (with more than one sequence) lengths drawn in
    [bound/16, bound] with the bound reached."""
    if B == 1:
        return {"equal": [ctx]}
    g = torch.Generator().manual_seed(seed)
    varied = torch.randint(max(lo_min, ctx // 16), ctx + 1, (B,), generator=g).tolist()
    varied[0] = ctx
    return {"equal": [ctx] * B, "varied": varied}


def decode_candidates(B, ctx):
    ntiles = -(-ctx // 16)
    out = []
    for S in SPLITS:
        if S > 1 and S > max(1, ntiles // 4):
            continue
        for W in WAVES:
            for V in VARIANTS:
                if S == 1 and V == 6:
                    continue
                if B == 1 and V == 6:  # one sequence: the even grid is the static grid
                    continue
                out.append((S, W, V if S > 1 else 0))
    return out


def sweep_decode(torch, pa, workloads, dev, results, groups):
    for G in groups:
        table = results.setdefault("decode", {}).setdefault(f"g{G}", {})
        for units in UNIT_BUCKETS:
            B = units // 8
            for ctx in CTX_BUCKETS:
                if B * ctx > MAX_TOKENS:
                    continue
                key = f"{units}x{ctx}"
                if key in table:
                    continue
                times = {}
                for mix, contexts in _mixes(torch, B, ctx, units * 131 + ctx + G).items():
                    spec = _spec(workloads, f"sw_g{G}_{key}_{mix}", contexts, [1] * B, 7, G=G)
                    b = workloads.generate(spec, dev, fill="zero")
                    pools = _pools(b, _copies(sum(contexts) * 4096))
                    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, B, spec.scale, ctx, 1)
                    out = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)
                    for S, W, V in decode_candidates(B, ctx):
                        t = pa.Tiles(16, S, W, 1, V)
                        ws = torch.zeros(max(pa.workspace_size(pb, t), 256),
                                         dtype=torch.uint8, device=dev)
                        fns = [(lambda kp=kp, vp=vp, t=t, ws=ws: pa.decode(
                            b.q, kp, vp, b.block_tables, b.context_lens, spec.scale, ctx,
                            out=out, tiles=t, workspace=ws, problem=pb)) for kp, vp in pools]
                        us = _time_graph(torch, fns)
                        times.setdefault(f"{S},{W},{V}", {})[mix] = round(us, 2)
                    del b, pools
                    torch.cuda.empty_cache()
                table[key] = times
                log(f"decode G={G} units={units} ctx={ctx}: {len(times)} candidates, "
                    f"pick {choose_decode_row(table, units)[ctx]}")


def sweep_prefill(torch, pa, workloads, dev, results):
    for D in PF_DIMS:
        table = results.setdefault("prefill", {}).setdefault(f"d{D}", {})
        q_tile = (128 if D == 256 else 256) // 4  # G = 4, 8 KV heads
        for wgs in PF_WG_BUCKETS:
            tiles = max(1, wgs // 8)
            for ctx in PF_CTX_BUCKETS:
                key = f"{wgs}x{ctx}"
                if key in table:
                    continue
                q = min(ctx, 2048)
                B = max(1, -(-tiles * q_tile // q))
                if B * ctx > MAX_TOKENS:
                    continue
                qlen = min(q, tiles * q_tile // B) or q_tile
                spec = _spec(workloads, f"swp_d{D}_{key}", [ctx] * B, [qlen] * B, 9, D=D)
                b = workloads.generate(spec, dev, fill="zero")
                pools = _pools(b, _copies(B * ctx * 32 * D))
                pb = pa.make_problem(b.q, b.k_pool, b.block_tables, B, spec.scale, ctx, qlen)
                out = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)
                times = {}
                for ts in PF_TILE_SPLITS:
                    t, _ = pa.select_tiles(pb)
                    t.tile_splits = ts
                    ws = torch.zeros(max(pa.workspace_size(pb, t), 256), dtype=torch.uint8,
                                     device=dev)
                    fns = [(lambda kp=kp, vp=vp, t=t, ws=ws: pa.prefill(
                        b.q, b.query_start_loc, kp, vp, b.block_tables, b.context_lens,
                        spec.scale, ctx, qlen, out=out, tiles=t, workspace=ws, problem=pb))
                        for kp, vp in pools]
                    times[str(ts)] = round(_time_graph(torch, fns), 2)
                table[key] = times
                log(f"prefill D={D} wgs={wgs} ctx={ctx} (B={B} q={qlen}): {times}")
                del b, pools
                torch.cuda.empty_cache()


def sweep_short(torch, pa, workloads, dev, results):
    res = results.setdefault("short", {})
    for D, wide in SHORT_KEYS:
        hkv = 1 if wide else 8
        for G, q in SHORT_SHAPES[wide][D]:
            shape = f"d{D}_w{wide}_g{G}_q{q}"
            per_shape = res.setdefault(shape, {})
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
                    times = {}
                    mixes = _mixes(torch, B, ctx, units * 137 + ctx + G + D + q, lo_min=q)
                    for mix, contexts in mixes.items():
                        spec = _spec(workloads, f"sws_{shape}_{key}_{mix}", contexts, [q] * B,
                                     11, G=G, hkv=hkv, D=D)
                        b = workloads.generate(spec, dev, fill="zero")
                        pools = _pools(b, _copies(sum(contexts) * hkv * D * 4))
                        pb = pa.make_problem(b.q, b.k_pool, b.block_tables, B, spec.scale, ctx, q)
                        out = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)
                        for S in SHORT_SPLITS:
                            if S > 1 and S > max(1, -(-ctx // 16) // 4):
                                continue
                            t, _ = pa.select_tiles(pb)
                            t.num_splits = S
                            ws = torch.zeros(max(pa.workspace_size(pb, t), 256),
                                             dtype=torch.uint8, device=dev)
                            if q == 1:
                                fns = [(lambda kp=kp, vp=vp, t=t, ws=ws: pa.decode(
                                    b.q, kp, vp, b.block_tables, b.context_lens, spec.scale, ctx,
                                    out=out, tiles=t, workspace=ws, problem=pb))
                                    for kp, vp in pools]
                            else:
                                fns = [(lambda kp=kp, vp=vp, t=t, ws=ws: pa.prefill(
                                    b.q, b.query_start_loc, kp, vp, b.block_tables,
                                    b.context_lens, spec.scale, ctx, q, out=out, tiles=t,
                                    workspace=ws, problem=pb)) for kp, vp in pools]
                            times.setdefault(str(S), {})[mix] = round(_time_graph(torch, fns), 2)
                        del b, pools
                        torch.cuda.empty_cache()
                    per_shape[key] = times
                    log(f"short {shape} units={units} ctx={ctx}: {len(times)} bounds")


def _scores(per_cand):
    """Worst time relative to the best of each mix (or shape and mix)."""
    best = {}
    for per in per_cand.values():
        for m, us in per.items():
            best[m] = min(best.get(m, 1e30), us)
    return {c: max(per[m] / best[m] for m in per) for c, per in per_cand.items()
            if len(per) == len(best)}


def _pick(score, prev_split, split_of, preferred):
    """The choice rule: ties within NEAR_TIE of the best; the preferred
    candidates among them if any; then the smallest split not below
    prev_split; else (a measured non-monotone step) the best."""
    best = min(score, key=score.get)
    tie = [c for c in score if score[c] <= score[best] * NEAR_TIE]
    pref = [c for c in tie if preferred(c)] or tie
    mono = [c for c in pref if split_of(c) >= prev_split]
    if mono:
        return min(mono, key=lambda c: (split_of(c), score[c]))
    return best


def choose_decode_row(table, units):
    """Choices of one units row of one group's decode table, context by
    context: {ctx: (S, W, V)}."""
    dflt_v = 6 if units > 8 else 2
    prev, row = 1, {}
    for ctx in CTX_BUCKETS:
        times = table.get(f"{units}x{ctx}")
        if not times:
            continue
        score = _scores(times)
        c = _pick(score, prev, lambda k: int(k.split(",")[0]),
                  lambda k: k.split(",")[1] == "4" and int(k.split(",")[2]) in (dflt_v, 0))
        row[ctx] = tuple(int(x) for x in c.split(","))
        prev = row[ctx][0]
    return row


def choose_short(results):
    """{(D, wide): {units: {ctx: S}}}: per bucket, the bound with the least
    worst relative time over the key's shapes and both mixes."""
    out = {}
    for D, wide in SHORT_KEYS:
        shapes = [f"d{D}_w{wide}_g{G}_q{q}" for G, q in SHORT_SHAPES[wide][D]]
        per_key = {}
        for units in SHORT_UNIT_BUCKETS:
            prev, row = 1, {}
            for ctx in SHORT_CTX_BUCKETS:
                key = f"{units}x{ctx}"
                merged = {}
                for sh in shapes:
                    for S, per in results.get("short", {}).get(sh, {}).get(key, {}).items():
                        for m, us in per.items():
                            merged.setdefault(S, {})[f"{sh}/{m}"] = us
                if not merged:
                    continue
                c = _pick(_scores(merged), prev, int, lambda k: True)
                row[ctx] = int(c)
                prev = row[ctx]
            per_key[units] = row
        out[(D, wide)] = per_key
    return out


def choose_prefill(results):
    """{D: {wgs: {ctx: tile_splits}}}"""
    out = {}
    for D in PF_DIMS:
        table = results.get("prefill", {}).get(f"d{D}", {})
        per_d = {}
        for wgs in PF_WG_BUCKETS:
            row = {}
            for ctx in PF_CTX_BUCKETS:
                times = table.get(f"{wgs}x{ctx}")
                if times:
                    best = min(times.values())
                    tie = [k for k, v in times.items() if v <= best * NEAR_TIE]
                    row[ctx] = min(int(k) for k in tie)  # fewer partials on a tie
            per_d[wgs] = row
        out[D] = per_d
    return out


def emit_header(results, path=GEN_HEADER):
    groups = [G for G in DECODE_GROUPS if f"g{G}" in results.get("decode", {})] or [4]
    lines = [
        "// Generated by paged_gqa_attention_pa_amd/tune/sweep.py from the gfx950",
        "// measurements in tune/sweep_gfx950.json; regenerate, do not edit.",
        "// Every entry: the launch shape whose worst time relative to the best, over",
        "// equal and spread context lengths (and the key's shapes), is within 2% of",
        "// the least, preferring the default shape and then the smallest split count",
        "// not below the shorter-context bucket's.  0 marks a bucket not swept.",
        "#pragma once",
        "",
        "namespace pa {",
        "namespace gen {",
        "",
        "// Decode kernels (head dim 128): {num_splits, waves, variant} per",
        "// (G, units = num_seqs * num_kv_heads, context bound).",
        f"constexpr int kDecodeGroups[] = {{{', '.join(map(str, groups))}}};",
        f"constexpr int kUnitBuckets[] = {{{', '.join(map(str, UNIT_BUCKETS))}}};",
        f"constexpr int kCtxBuckets[] = {{{', '.join(map(str, CTX_BUCKETS))}}};",
        f"constexpr unsigned short kDecode[{len(groups)}][{len(UNIT_BUCKETS)}]"
        f"[{len(CTX_BUCKETS)}][3] = {{",
    ]
    for G in groups:
        table = results.get("decode", {}).get(f"g{G}", {})
        lines.append(f"    {{  // G = {G}")
        for u in UNIT_BUCKETS:
            row = choose_decode_row(table, u)
            cells = ["{%d, %d, %d}" % row[c] if c in row else "{0, 0, 0}" for c in CTX_BUCKETS]
            lines.append("        {" + ", ".join(cells) + "},")
        lines.append("    },")
    lines += ["};", ""]
    short = choose_short(results)
    lines += [
        "// Short query runs (the short-run kernel): split bound per (head dim,",
        "// wide = G >= 16) key and (units, context bound) bucket, over the shapes",
        "// (G, tokens): " + "; ".join(
            f"D {D} {'wide' if w else 'narrow'} " + ", ".join(f"({g}, {q})" for g, q in
                                                           SHORT_SHAPES[w][D])
            for D, w in SHORT_KEYS) + ".",
        f"constexpr int kShortKeys[][2] = {{{', '.join('{%d, %d}' % k for k in SHORT_KEYS)}}};",
        f"constexpr int kShortUnitBuckets[] = {{{', '.join(map(str, SHORT_UNIT_BUCKETS))}}};",
        f"constexpr int kShortCtxBuckets[] = {{{', '.join(map(str, SHORT_CTX_BUCKETS))}}};",
        f"constexpr unsigned short kShortSplits[{len(SHORT_KEYS)}][{len(SHORT_UNIT_BUCKETS)}]"
        f"[{len(SHORT_CTX_BUCKETS)}] = {{",
    ]
    for k in SHORT_KEYS:
        lines.append(f"    {{  // head dim {k[0]}, {'wide' if k[1] else 'narrow'} G")
        for u in SHORT_UNIT_BUCKETS:
            row = short[k].get(u, {})
            lines.append("        {" + ", ".join(str(row.get(c, 0)) for c in SHORT_CTX_BUCKETS)
                         + "},")
        lines.append("    },")
    lines += ["};", ""]
    pf = choose_prefill(results)
    lines += [
        "// Prefill: tile_splits per (head dim, query-tile workgroups, context bound).",
        f"constexpr int kPfDims[] = {{{', '.join(map(str, PF_DIMS))}}};",
        f"constexpr int kPfWgBuckets[] = {{{', '.join(map(str, PF_WG_BUCKETS))}}};",
        f"constexpr int kPfCtxBuckets[] = {{{', '.join(map(str, PF_CTX_BUCKETS))}}};",
        f"constexpr unsigned char kPrefillTileSplits[{len(PF_DIMS)}][{len(PF_WG_BUCKETS)}]"
        f"[{len(PF_CTX_BUCKETS)}] = {{",
    ]
    for D in PF_DIMS:
        lines.append(f"    {{  // head dim {D}")
        for w in PF_WG_BUCKETS:
            row = pf[D].get(w, {})
            lines.append("        {" + ", ".join(str(row.get(c, 0)) for c in PF_CTX_BUCKETS)
                         + "},")
        lines.append("    },")
    lines += ["};", "", "}  // namespace gen", "}  // namespace pa", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))
    log(f"wrote {path}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out-json", default=DEFAULT_JSON)
    ap.add_argument("--emit-only", action="store_true", help="regenerate the header from JSON")
    ap.add_argument("--part", choices=["decode", "short", "prefill"], action="append")
    ap.add_argument("--groups", type=int, nargs="*", default=DECODE_GROUPS)
    ap.add_argument("--no-header", action="store_true")
    args = ap.parse_args()
    results = {}
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
        parts = args.part or ["decode", "short", "prefill"]
        try:
            if "decode" in parts:
                sweep_decode(torch, pa, workloads, dev, results, args.groups)
            if "short" in parts:
                sweep_short(torch, pa, workloads, dev, results)
            if "prefill" in parts:
                sweep_prefill(torch, pa, workloads, dev, results)
        finally:
            with open(args.out_json, "w") as f:
                json.dump(results, f, indent=0, sort_keys=True)
            log(f"sweep {time.time() - t0:.0f} s, results in {args.out_json}")
    if not args.no_header:
        emit_header(results)


if __name__ == "__main__":
    main()
