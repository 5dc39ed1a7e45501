"""Replay the launch shapes the tile table chose, one bucket after another,
for a profiler to attribute kernel time and HBM bytes to each chosen entry.

    rocprofv3 --kernel-trace --stats -f csv -d OUT -o run -- \\
        python3 -m paged_gqa_attention_pa_amd.tune.profile_entries
    rocprofv3 --pmc FETCH_SIZE -f csv -d OUT -o run -- \\
        python3 -m paged_gqa_attention_pa_amd.tune.profile_entries --calibrate-copy 256

For every decode bucket listed below (G, units = num_seqs * 8 KV heads,
context bound, all contexts equal to the bound) it builds a seeded
synthetic batch the way the sweep does (pools 2.5x the pages in use,
shuffled), takes the launch shape pa_select_tiles returns, and calls
pa_decode once per K/V pool copy, with enough copies that the calls of a
bucket move at least 512 MiB of K/V (no call is served by the Infinity
Cache), `--rounds` times.  Each bucket prints one JSON line, in launch
order: the chosen tiles, the calls made and the algorithmic K/V bytes per
call, so a trace's decode dispatches can be assigned to buckets in order.
`--calibrate-copy MIB` ends with four device copies of that size, whose
counter readings scale FETCH_SIZE / WRITE_SIZE to bytes.
"""
import argparse
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

# (G, units, context bound) of the decode table
BUCKETS = [(G, units, ctx) for G in (1, 4, 8) for units in (8, 64, 512)
           for ctx in (1024, 8192, 32768) if (units // 8) * ctx <= 1 << 21]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--rounds", type=int, default=3, help="calls per pool copy and bucket")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="end with four device copies of MIB MiB (counter calibration)")
    args = ap.parse_args(argv)

    import torch
    from paged_gqa_attention_pa_amd import pa, workloads
    from paged_gqa_attention_pa_amd.tune import sweep

    dev = torch.device("cuda:0")
    for G, units, ctx in BUCKETS:
        B = units // 8
        spec = sweep._spec(workloads, f"pe_g{G}_{units}x{ctx}", [ctx] * B, [1] * B, 7, G=G)
        b = workloads.generate(spec, dev, fill="zero")
        kv_bytes = B * ctx * 8 * 128 * 2 * 2
        pools = sweep._pools(b, sweep._copies(kv_bytes))
        pb = pa.make_problem(b.q, b.k_pool, b.block_tables, B, spec.scale, ctx, 1)
        tiles, ws_bytes = pa.select_tiles(pb)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        out = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)
        calls = 0
        for _ in range(args.rounds):
            for kp, vp in pools:
                pa.decode(b.q, kp, vp, b.block_tables, b.context_lens, spec.scale, ctx, out=out,
                          tiles=tiles, workspace=ws, problem=pb)
                calls += 1
        torch.cuda.synchronize()
        print(json.dumps({"bucket": {"G": G, "units": units, "ctx": ctx, "num_seqs": B},
                          "tiles": {"num_splits": tiles.num_splits,
                                    "waves_per_wg": tiles.waves_per_wg,
                                    "variant": tiles.variant},
                          "calls": calls, "pool_copies": len(pools),
                          "kv_bytes_per_call": kv_bytes}), flush=True)
        del b, pools, ws, out
        torch.cuda.empty_cache()
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 4}), flush=True)


if __name__ == "__main__":
    main()
