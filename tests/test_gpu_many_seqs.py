"""GPU parity for calls with many sequences, every row against the oracle.

Each workgroup of the query-tile path finds its (sequence, tile) by a scan of
query_start_loc in chunks of one workgroup's threads (512 sequences), the
tile merge repeats that scan, the even-work decode grid scans every context
length, and the short-run units are laid out per sequence: with 1,000-2,000
sequences every one of those scans runs over several chunks, which the
smaller batches of the other tests never reach.  Lengths are drawn from
seeded generators: empty contexts, single keys and page-boundary lengths
are among them.
"""
import numpy as np
import pytest
import torch

from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_parity import compare, dev, log, run_decode, run_prefill  # noqa: F401

pytestmark = pytest.mark.gpu


def _decode_lengths(n, seed, hi):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(0, hi + 1, n)
    ctx[rng.random(n) < 0.05] = 0
    ctx[:4] = [0, 1, 16, 17]
    return [int(c) for c in ctx]


@pytest.mark.parametrize("splits,variant", [(None, None), (1, 0), (3, 2), (2, 6), (8, 6)],
                         ids=["table", "static1", "static3", "even2", "even8"])
def test_decode_many_sequences(dev, splits, variant):
    """2,000 single-token sequences, contexts 0..120, on the table's launch
    shape and on forced static and even-work grids."""
    log(f"[decode 2000 sequences splits={splits} variant={variant}]")
    ctx = _decode_lengths(2000, 41, 120)
    spec = workloads.small_spec("many_dec", seed=41, contexts=ctx, queries=[1] * len(ctx))
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_decode(b, dt, splits, variant=variant)
        compare(b, out, lse, label=f"decode 2000 seqs S={splits} v={variant} {dt}")


def _mixed_lengths(n, seed, decode_frac, q_hi, prefix_hi):
    rng = np.random.default_rng(seed)
    ql, ctx = [], []
    for _ in range(n):
        if rng.random() < decode_frac:
            q = 1
        else:
            q = int(rng.integers(2, q_hi + 1))
        prefix = int(rng.integers(0, prefix_hi + 1))
        ql.append(q)
        ctx.append(prefix + q)
    return ctx, ql


@pytest.mark.parametrize("mode", ["bench_launch", "tile_splits", "even_decode_rows"])
def test_mixed_many_sequences(dev, mode):
    """1,200 sequences, 60% single-token (decode rows) and the rest chunks
    of 2..40 query tokens over prefixes of 0..200 keys, in one pa_prefill
    call: the table's launch as the benchmark makes it (bf16, no LSE), query
    tiles split in two runs, and decode rows on the even-work grid."""
    log(f"[mixed 1200 sequences {mode}]")
    ctx, ql = _mixed_lengths(1200, 43, 0.6, 40, 200)
    spec = workloads.small_spec("many_mix", seed=43, contexts=ctx, queries=ql,
                                decode_layout=False)
    b = workloads.generate(spec, dev)
    if mode == "bench_launch":
        out, lse = run_prefill(b, torch.bfloat16, with_lse=False)
    elif mode == "tile_splits":
        out, lse = run_prefill(b, torch.float32, tile_splits=2, stale_workspace=True)
    else:
        out, lse = run_prefill(b, torch.float32, splits=4, variant=7)
    compare(b, out, lse, label=f"mixed 1200 seqs {mode}")


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8)], ids=["g4", "g8"])
def test_short_runs_many_sequences(dev, hq, hkv):
    """1,100 sequences of 2..6 query tokens (speculative-decode verification)
    over prefixes of 0..400 keys."""
    log(f"[short runs 1100 sequences G={hq // hkv}]")
    ctx, ql = _mixed_lengths(1100, 47 + hq, 0.0, 6, 400)
    spec = workloads.small_spec("many_short", seed=47 + hq, contexts=ctx, queries=ql,
                                num_q_heads=hq, num_kv_heads=hkv, decode_layout=False)
    b = workloads.generate(spec, dev)
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                         b.max_context_len, b.max_query_len)
    tiles, _ = pa.select_tiles(pb)
    assert tiles.q_tokens_per_tile == b.max_query_len, "not the short-run path"
    out, lse = run_prefill(b, torch.bfloat16)
    compare(b, out, lse, label=f"short runs 1100 seqs G={hq // hkv} bf16")
    out, lse = run_prefill(b, torch.float32, splits=3, stale_workspace=True)
    compare(b, out, lse, label=f"short runs 1100 seqs G={hq // hkv} f32 S=3")
