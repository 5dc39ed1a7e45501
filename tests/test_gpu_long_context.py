"""GPU parity at contexts of 128k keys, every row against the oracle.

At 131,072 keys a decode unit is 8,192 tiles (the table then cuts it into
its largest split counts), and a query tile walks its keys in four windows of
the LDS page-offset window (2,048 16-key blocks each, 1,024 at head dim 256,
so eight there), restaging it three times (seven).  The other tests stop at
40,000 keys.
"""
import pytest
import torch

from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_parity import (compare, dev, log, oracle_reference, run_decode,  # noqa: F401
                             run_prefill)

pytestmark = pytest.mark.gpu

LONG = 131072

_REFERENCE = {}  # oracle outputs per batch name: several launches compare against one


def _reference(b):
    if b.spec.name not in _REFERENCE:
        _REFERENCE[b.spec.name] = oracle_reference(b)
    return _REFERENCE[b.spec.name]


@pytest.mark.parametrize("splits,variant", [(None, None), (256, 2), (64, 0), (16, 6)],
                         ids=["table", "static256", "fused64", "even16"])
def test_decode_long_context(dev, splits, variant):
    """Two sequences of 131,072 and 70,001 keys beside a short one."""
    log(f"[decode 128k splits={splits} variant={variant}]")
    spec = workloads.small_spec("long_dec", seed=61, contexts=[LONG, 70001, 300],
                                queries=[1, 1, 1])
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_decode(b, dt, splits, variant=variant)
        compare(b, out, lse, label=f"decode 128k S={splits} v={variant} {dt}")


@pytest.mark.parametrize("mode", ["bench_launch", "f32_lse", "tile_splits8"])
def test_prefill_chunk_long_prefix(dev, mode):
    """A 48-token causal chunk at the end of a 131,072-key context, a
    40-token chunk over 70,000 keys and a single-token row: as the benchmark
    launches it (bf16, no LSE), with fp32 output and LSE, and with each query
    tile's keys cut into eight runs."""
    log(f"[prefill chunk at 128k {mode}]")
    spec = workloads.small_spec("long_pre", seed=67, contexts=[LONG, 70000, 5000],
                                queries=[48, 40, 1], decode_layout=False)
    b = workloads.generate(spec, dev)
    if mode == "bench_launch":
        out, lse = run_prefill(b, torch.bfloat16, with_lse=False)
    elif mode == "f32_lse":
        out, lse = run_prefill(b, torch.float32)
    else:
        out, lse = run_prefill(b, torch.float32, tile_splits=8, stale_workspace=True)
    compare(b, out, lse, label=f"prefill 128k {mode}", reference=_reference(b))


def test_short_runs_long_context(dev):
    """Speculative-decode verification (4 and 7 query tokens) over 131,072
    and 90,000 keys."""
    log("[short runs at 128k]")
    spec = workloads.small_spec("long_short", seed=71, contexts=[LONG, 90000],
                                queries=[4, 7], decode_layout=False)
    b = workloads.generate(spec, dev)
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                         b.max_context_len, b.max_query_len)
    tiles, _ = pa.select_tiles(pb)
    assert tiles.q_tokens_per_tile == b.max_query_len, "not the short-run path"
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_prefill(b, dt)
        compare(b, out, lse, label=f"short runs 128k {dt}")


@pytest.mark.parametrize("page", [16, 256])
def test_head_dim_256_long_prefix(dev, page):
    """Head dim 256 query tiles (1,024-block window, so seven restagings) on
    a 16-token chunk at the end of 131,072 keys, in pages of 16 and 256
    slots."""
    log(f"[prefill D=256 at 128k, page {page}]")
    spec = workloads.small_spec("long_d256", seed=73 + page, contexts=[LONG, 300],
                                queries=[16, 20], head_dim=256, page_size=page,
                                decode_layout=False)
    b = workloads.generate(spec, dev)
    out, lse = run_prefill(b, torch.float32)
    compare(b, out, lse, label=f"prefill D=256 128k page {page}")
