"""GPU parity of short query runs (speculative-decode verification) through
pa_prefill, against the fp64 oracle.

A batch whose longest query run has 2 <= q and q * G <= 64 takes the
short-run kernel: each (sequence, kv head) unit is one Q-block of q tokens x
G heads, streamed with the decode path's even-work grid, and units cut into
several pieces are merged by log-sum-exp.  Tolerances are those of the other
parity tests; the indexing cases must match bit for bit.
"""
import numpy as np
import pytest
import torch

from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_parity import (_dominant_batch, _permuted, compare, dev, log,  # noqa: F401
                             run_decode, run_prefill)

pytestmark = pytest.mark.gpu

VERIFY_CASES = [
    # (name, contexts, query lens, Hq, Hkv, causal)
    ("q4", [5, 16, 17, 300, 1000, 4100], [4, 4, 4, 4, 4, 4], 32, 8, True),
    ("ragged_q", [64, 2049, 33, 700, 8, 1, 16], [2, 3, 5, 8, 8, 1, 16], 32, 8, True),
    ("q16_g4", [16, 100, 3000], [16, 16, 9], 32, 8, True),
    ("whole_context", [2, 7, 16], [2, 7, 16], 32, 8, True),
    ("empty_seqs", [100, 0, 50, 9], [3, 0, 2, 0], 32, 8, True),
    ("g1_q16", [500, 17, 2000], [16, 11, 2], 8, 8, True),
    ("g2_q16", [500, 17, 2000], [16, 11, 2], 16, 8, True),
    ("g8_q8", [500, 17, 2000], [8, 5, 2], 64, 8, True),
    ("g16_q4", [500, 17, 2000], [4, 3, 2], 16, 1, True),
    ("noncausal", [300, 45, 1000], [6, 4, 8], 32, 8, False),
    ("long_context", [40000, 300], [4, 3], 32, 8, True),
    # 40 sequences x 8 kv heads x 16 rows: enough rows for the per-unit merge
    ("many_units", [17 + (97 * i) % 3000 for i in range(40)], [1 + i % 4 for i in range(40)],
     32, 8, True),
]


@pytest.mark.parametrize("name,ctx,ql,hq,hkv,causal", VERIFY_CASES,
                         ids=[c[0] for c in VERIFY_CASES])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_verify_small(dev, name, ctx, ql, hq, hkv, causal, out_dtype):
    log(f"[verify {name} {out_dtype}]")
    spec = workloads.small_spec(f"ver_{name}", seed=800 + sum(ql) + hq, contexts=ctx, queries=ql,
                                num_q_heads=hq, num_kv_heads=hkv, causal=causal,
                                decode_layout=False)
    b = workloads.generate(spec, dev)
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                         b.max_context_len, b.max_query_len, causal=causal)
    tiles, _ = pa.select_tiles(pb)
    assert tiles.q_tokens_per_tile == b.max_query_len, "not the short-run path"
    out, lse = run_prefill(b, out_dtype)
    compare(b, out, lse, label=f"verify {name}")


@pytest.mark.parametrize("splits", [1, 3, 64])
def test_verify_split_counts_stale_workspace(dev, splits):
    """Forced split counts over a workspace of 0xFF bytes (NaN partials,
    piece counts of -1): units cut into up to splits + 1 pieces."""
    log(f"[verify splits={splits} stale workspace]")
    spec = workloads.small_spec("ver_split", seed=820 + splits, contexts=[4000, 33, 2500, 16, 900],
                                queries=[4, 2, 8, 3, 5], decode_layout=False, pool_slack=20)
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                             b.max_context_len, b.max_query_len, out_dtype=dt)
        t, _ = pa.select_tiles(pb)
        t.num_splits = splits
        ws = torch.full((pa.workspace_size(pb, t),), 0xFF, dtype=torch.uint8, device=dev)
        lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=dev)
        out = pa.prefill(b.q, b.query_start_loc, b.k_pool, b.v_pool, b.block_tables,
                         b.context_lens, spec.scale, b.max_context_len, b.max_query_len,
                         out_dtype=dt, lse=lse, tiles=t, workspace=ws, problem=pb)
        torch.cuda.synchronize()
        compare(b, out, lse, label=f"verify S={splits} {dt}")


def test_verify_dominant_logit_bitexact(dev):
    log("[verify dominant logit]")
    L, q = 300, 4
    tstars = [0, 15, 16, 200, 296]  # all <= L - q: every row of the run sees t*
    b = _dominant_batch(dev, tstars, L, prefill_q=q)
    for dt in (torch.bfloat16, torch.float32):
        out, _ = run_prefill(b, dt)
        for s, t in enumerate(tstars):
            page = int(b.block_tables[s, t // 16])
            want = b.v_pool[page, t % 16].repeat_interleave(4, dim=0).to(dt)
            got = out[s * q:(s + 1) * q]
            ok = (torch.equal(got.view(torch.int16), want.view(torch.int16).expand_as(got))
                  if dt == torch.bfloat16 else torch.equal(got, want.expand_as(got)))
            assert ok, f"seq {s} t*={t} {dt}"


def test_verify_page_permutation_and_nan_bitexact(dev):
    log("[verify permutation / NaN poison]")
    spec = workloads.small_spec("vperm", seed=47, contexts=[301, 77, 40, 1000], queries=[4, 7, 1, 2],
                                pool_slack=30, decode_layout=False)
    b = workloads.generate(spec, dev, fill="nan")
    bz = workloads.generate(spec, dev, fill="zero")
    o1, l1 = run_prefill(b, torch.float32)
    o2, l2 = run_prefill(_permuted(b), torch.float32)
    o3, l3 = run_prefill(bz, torch.float32)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_verify_rows_match_decode(dev):
    """Row i of a causal run over L keys equals a decode step over the first
    L - q + i + 1 keys of the same pages (fp32 outputs, both paths' own
    rounding: agreement to the fp32 tolerance, not bits)."""
    log("[verify rows vs decode]")
    L, q = 3000, 6
    spec = workloads.small_spec("vdec", seed=48, contexts=[L], queries=[q], decode_layout=False)
    b = workloads.generate(spec, dev)
    out, _ = run_prefill(b, torch.float32)
    for i in range(q):
        lens = torch.tensor([L - q + i + 1], dtype=torch.int32, device=dev)
        o = pa.decode(b.q[i:i + 1].contiguous(), b.k_pool, b.v_pool, b.block_tables, lens,
                      spec.scale, L - q + i + 1, out_dtype=torch.float32)
        torch.cuda.synchronize()
        err = float((o[0] - out[i]).abs().max())
        assert err <= 2e-3, f"row {i}: {err}"


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 1)], ids=["g4", "g16"])
@pytest.mark.parametrize("variant", [2, 6], ids=["static", "even"])
@pytest.mark.parametrize("splits", [1, 4])
def test_prefill_single_token_batch(dev, hq, hkv, variant, splits):
    """pa_prefill on a batch whose sequences have at most one query token
    (one with none) runs on the decode kernels."""
    log(f"[prefill single-token batch G={hq // hkv} variant={variant} S={splits}]")
    spec = workloads.small_spec("pre_q1", seed=830 + hq + splits, contexts=[700, 50, 3000, 1, 16],
                                queries=[1, 0, 1, 1, 1], num_q_heads=hq, num_kv_heads=hkv,
                                decode_layout=False)
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                             b.max_context_len, 1, out_dtype=dt)
        t, _ = pa.select_tiles(pb)
        t.num_splits, t.variant = splits, variant
        ws = torch.full((max(pa.workspace_size(pb, t), 16),), 0xFF, dtype=torch.uint8, device=dev)
        lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=dev)
        out = pa.prefill(b.q, b.query_start_loc, b.k_pool, b.v_pool, b.block_tables,
                         b.context_lens, spec.scale, b.max_context_len, 1, out_dtype=dt,
                         lse=lse, tiles=t, workspace=ws, problem=pb)
        torch.cuda.synchronize()
        compare(b, out, lse, label=f"single-token prefill G={hq // hkv} v{variant} S={splits} {dt}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (64, 8), (16, 1)],
                         ids=["g1", "g4", "g8", "g16"])
@pytest.mark.parametrize("splits", [1, 4, 33])
def test_decode_short_run_variant(dev, hq, hkv, splits):
    """Variant bit 3 puts decode rows (G <= 16) on the short-run kernel, in
    pa_decode and in a single-token pa_prefill; the workspace starts stale."""
    log(f"[decode on the short-run kernel G={hq // hkv} S={splits}]")
    ctx = [700, 33, 1, 0, 2049, 16, 4100]
    spec = workloads.small_spec("dec_short", seed=880 + hq + splits, contexts=ctx,
                                queries=[1] * len(ctx), num_q_heads=hq, num_kv_heads=hkv)
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                             b.max_context_len, 1, out_dtype=dt)
        t, _ = pa.select_tiles(pb)
        t.num_splits, t.waves_per_wg, t.variant = splits, 4, t.variant | 14
        ws = torch.full((pa.workspace_size(pb, t),), 0xFF, dtype=torch.uint8, device=dev)
        out, lse = run_decode(b, dt, splits, waves=4, variant=t.variant, workspace=ws)
        compare(b, out, lse, label=f"short-run decode G={hq // hkv} S={splits} {dt}")
    # the same rows through pa_prefill's packed layout
    spec = workloads.small_spec("pre_short", seed=890 + hq + splits, contexts=ctx,
                                queries=[1, 0, 1, 1, 1, 1, 1], num_q_heads=hq,
                                num_kv_heads=hkv, decode_layout=False)
    b = workloads.generate(spec, dev)
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                         b.max_context_len, 1)
    t, _ = pa.select_tiles(pb)
    t.num_splits, t.waves_per_wg, t.variant = splits, 4, t.variant | 14
    ws = torch.full((pa.workspace_size(pb, t),), 0xFF, dtype=torch.uint8, device=dev)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=dev)
    out = pa.prefill(b.q, b.query_start_loc, b.k_pool, b.v_pool, b.block_tables,
                     b.context_lens, spec.scale, b.max_context_len, 1, lse=lse, tiles=t,
                     workspace=ws, problem=pb)
    torch.cuda.synchronize()
    compare(b, out, lse, label=f"short-run single-token prefill G={hq // hkv} S={splits}")


# ---------------------------------------------------- 32 heads per KV head ----

G32_DECODE = [1, 15, 16, 17, 300, 1000, 0, 2049]


@pytest.mark.parametrize("splits", [None, 1, 3, 64])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_g32_decode(dev, splits, out_dtype):
    """pa_decode with 32 query heads on one KV head: one token of 32 heads is
    two 16-row blocks of the short-run kernel (decode layout, no
    query_start_loc)."""
    log(f"[decode G=32 S={splits} {out_dtype}]")
    spec = workloads.small_spec("g32_dec", seed=850, contexts=G32_DECODE,
                                queries=[1] * len(G32_DECODE), num_q_heads=32, num_kv_heads=1)
    b = workloads.generate(spec, dev)
    out, lse = run_decode(b, out_dtype, splits)
    compare(b, out, lse, label=f"decode G=32 S={splits}")


@pytest.mark.parametrize("ctx", [1025, 20000, 70000])
@pytest.mark.parametrize("splits", [None, 256])
def test_single_unit_many_splits(dev, ctx, splits):
    """One sequence on one KV head (G = 32): the short-run table cuts the
    only unit into up to 128 pieces, and 256 forced; every row checked."""
    log(f"[single unit G=32 ctx={ctx} S={splits}]")
    spec = workloads.small_spec("g32_one", seed=870 + ctx % 97, contexts=[ctx], queries=[1],
                                num_q_heads=32, num_kv_heads=1)
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_decode(b, dt, splits)
        compare(b, out, lse, label=f"single unit ctx={ctx} S={splits} {dt}")


G32_PREFILL = [
    # (name, contexts, query lens): one-token rows, two-token runs (the
    # short-run kernel), chunks (query tiles of 8 tokens x 32 heads), a mix
    ("q1", [700, 50, 3000, 1, 16], [1, 0, 1, 1, 1]),
    ("q2", [700, 50, 3000, 2, 16], [2, 1, 2, 2, 1]),
    ("chunks", [300, 77, 1000], [140, 77, 31]),
    ("mixed", [900, 40, 260, 513], [1, 1, 100, 200]),
]


@pytest.mark.parametrize("name,ctx,ql", G32_PREFILL, ids=[c[0] for c in G32_PREFILL])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_g32_prefill(dev, name, ctx, ql, out_dtype):
    log(f"[prefill G=32 {name} {out_dtype}]")
    spec = workloads.small_spec(f"g32_{name}", seed=860 + sum(ql), contexts=ctx, queries=ql,
                                num_q_heads=32, num_kv_heads=1, decode_layout=False)
    b = workloads.generate(spec, dev)
    out, lse = run_prefill(b, out_dtype)
    compare(b, out, lse, label=f"prefill G=32 {name}")


# one case per (G, row blocks) the short-run path builds at head dim 128, and
# one just past it (128 rows: the query tiles)
ROW_BLOCK_CASES = [(g, q) for g, qs in [(1, [2, 20, 40, 100]), (2, [2, 12, 24, 60]),
                                        (4, [2, 8, 16, 32]), (8, [2, 4, 8, 16]),
                                        (16, [2, 4, 8]), (32, [2, 4])] for q in qs]


@pytest.mark.parametrize("g,q", ROW_BLOCK_CASES, ids=[f"G{g}_q{q}" for g, q in ROW_BLOCK_CASES])
def test_verify_every_row_block(dev, g, q):
    """Runs of q tokens x G heads = 16, 32 or 64 rows per unit (one, two or
    four row blocks; four share a tile stream between two wavefronts), and
    128 rows (query tiles), in fp32 and bf16."""
    hkv = 1 if g == 32 else 8 // min(g, 8) if g > 8 else 2
    hq = g * hkv
    log(f"[verify G={g} q={q} Hq={hq} Hkv={hkv}]")
    spec = workloads.small_spec(f"rb_g{g}_q{q}", seed=1100 + g + q, contexts=[q + 300, q + 5, 2000, q],
                                queries=[q, max(1, q // 2), 1, q], num_q_heads=hq,
                                num_kv_heads=hkv, decode_layout=False)
    b = workloads.generate(spec, dev)
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                         b.max_context_len, b.max_query_len)
    tiles, _ = pa.select_tiles(pb)
    assert tiles.kv_tile == (16 if q * g <= 64 else 32), "unexpected path"
    for dt in (torch.float32, torch.bfloat16):
        out, lse = run_prefill(b, dt)
        compare(b, out, lse, label=f"verify G={g} q={q} {dt}")
