"""GPU parity at head dims 64 and 256 against the fp64 oracle.

Decode and short query runs at these head dims run on the short-run kernel
(one Q-block per (sequence, kv head) unit, MFMA for both products); the
paged append copies rows of any head dim bit for bit.  Longer query runs
take the query-tile kernel (256-row Q-blocks at head dim 64, 128-row
Q-blocks of four wavefronts at 256).  In a mixed batch at these head dims
the single-token sequences are query tiles of their own, whose key runs the
library's launch splits.
"""
import numpy as np
import pytest
import torch

from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_append import append_and_check
from test_gpu_parity import compare, dev, log, run_decode, run_prefill  # noqa: F401

pytestmark = pytest.mark.gpu

DECODE_CTX = [1, 15, 16, 17, 300, 1000, 0, 2049]


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (64, 8), (32, 1)],
                         ids=["g1", "g4", "g8", "g32"])
@pytest.mark.parametrize("splits", [None, 1, 5])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_head_dim(dev, d, hq, hkv, splits, out_dtype):
    log(f"[decode D={d} G={hq // hkv} S={splits} {out_dtype}]")
    spec = workloads.small_spec(f"dec_d{d}", seed=900 + d + hq, contexts=DECODE_CTX,
                                queries=[1] * len(DECODE_CTX), num_q_heads=hq,
                                num_kv_heads=hkv, head_dim=d)
    b = workloads.generate(spec, dev)
    out, lse = run_decode(b, out_dtype, splits)
    compare(b, out, lse, label=f"decode D={d} G={hq // hkv} S={splits}")


SHORT_RUNS = [
    # (name, contexts, query lens, causal)
    ("q2", [64, 2049, 33, 700, 8, 1, 16], [2, 2, 2, 2, 2, 1, 2], True),
    ("q4_ragged", [5, 300, 1000, 4100, 0], [4, 3, 4, 1, 0], True),
    ("q8", [16, 100, 3000], [8, 8, 5], True),
    ("noncausal", [300, 45, 1000], [6, 4, 8], False),
]


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("name,ctx,ql,causal", SHORT_RUNS, ids=[c[0] for c in SHORT_RUNS])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_short_runs_head_dim(dev, d, name, ctx, ql, causal, out_dtype):
    log(f"[short runs D={d} {name} {out_dtype}]")
    spec = workloads.small_spec(f"sr_d{d}_{name}", seed=920 + d + sum(ql), contexts=ctx,
                                queries=ql, head_dim=d, causal=causal, decode_layout=False)
    b = workloads.generate(spec, dev)
    out, lse = run_prefill(b, out_dtype)
    compare(b, out, lse, label=f"short runs D={d} {name}")


@pytest.mark.parametrize("d", [64, 256])
def test_decode_head_dim_batch(dev, d):
    """A decode batch of 64 sequences with contexts U[128, 2048] at this head
    dim, every row checked."""
    log(f"[decode batch D={d}]")
    spec = workloads.WorkloadSpec(name=f"dec_b64_d{d}", seed=940 + d, pool_pages=12000,
                                  ctx_range=(128, 2048), num_draw=64, max_blocks=128,
                                  decode_layout=True, head_dim=d)
    b = workloads.generate(spec, dev)
    out, lse = run_decode(b, torch.bfloat16)
    compare(b, out, lse, label=f"decode batch D={d}")


@pytest.mark.parametrize("d", [64, 256])
def test_append_head_dim(dev, d):
    log(f"[append D={d}]")
    spec = workloads.small_spec(f"app_d{d}", seed=950 + d, contexts=[1, 15, 300, 1000, 33],
                                queries=[1, 15, 100, 1, 16], head_dim=d, pool_slack=9)
    b = workloads.generate(spec, dev)
    kn, vn = workloads.new_kv(b, seed=960 + d)
    append_and_check(b, kn, vn, f"append D={d}")


PREFILL_D64 = [
    # (name, contexts, query lens, causal)
    ("chunks", [300, 77, 1000, 33], [140, 77, 31, 33], True),
    ("tiles", [32, 64, 65, 200], [32, 64, 65, 129], True),
    ("noncausal", [300, 50], [100, 7], False),
    ("decode_rows", [900, 40, 260, 513], [1, 1, 100, 200], True),
    ("long_context", [40000, 300], [32, 20], True),
]


@pytest.mark.parametrize("name,ctx,ql,causal", PREFILL_D64, ids=[c[0] for c in PREFILL_D64])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_head_dim_64(dev, name, ctx, ql, causal, out_dtype):
    """Query tiles at head dim 64 (K and V staged by separate wavefront halves)."""
    log(f"[prefill D=64 {name} {out_dtype}]")
    spec = workloads.small_spec(f"pf64_{name}", seed=980 + sum(ql), contexts=ctx, queries=ql,
                                head_dim=64, causal=causal, decode_layout=False)
    b = workloads.generate(spec, dev)
    T = sum(ql) * spec.num_q_heads
    rows = None
    if T > 8192:
        rng = np.random.default_rng(3)
        rows = np.unique(np.concatenate([rng.choice(T, 4096, replace=False), [0, T - 1]]))
    out, lse = run_prefill(b, out_dtype)
    compare(b, out, lse, rows=rows, label=f"prefill D=64 {name}")


@pytest.mark.parametrize("ts", [2, 5])
def test_prefill_head_dim_64_tile_splits(dev, ts):
    log(f"[prefill D=64 tile splits {ts}]")
    spec = workloads.small_spec("pf64_ts", seed=990 + ts, contexts=[2100, 1500], queries=[300, 200],
                                head_dim=64, decode_layout=False)
    b = workloads.generate(spec, dev)
    rng = np.random.default_rng(ts)
    T = 500 * spec.num_q_heads
    rows = np.unique(np.concatenate([rng.choice(T, 4096, replace=False), [0, T - 1]]))
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_prefill(b, dt, tile_splits=ts, stale_workspace=True)
        compare(b, out, lse, rows=rows, label=f"prefill D=64 ts={ts} {dt}")


PREFILL_D256 = [
    # (name, contexts, query lens, causal, hq, hkv)
    ("chunks", [300, 77, 1000, 33], [140, 77, 31, 33], True, 32, 8),
    ("tiles", [32, 64, 65, 200], [32, 64, 65, 129], True, 32, 8),
    ("noncausal", [300, 50], [100, 7], False, 32, 8),
    # single-token sequences take the query tiles at head dim 256
    ("decode_rows", [900, 40, 260, 513], [1, 1, 100, 200], True, 32, 8),
    ("g1", [200, 90], [70, 90], True, 8, 8),
    ("g2", [200, 90], [70, 90], True, 16, 8),
    ("g8", [200, 90], [70, 90], True, 32, 4),
    ("g16", [200, 90], [70, 90], True, 16, 1),
    ("g32", [300, 77], [40, 9], True, 32, 1),
    # more than 1024 16-key blocks: the LDS window of block offsets (16k keys
    # at head dim 256) is restaged
    ("long_context", [20000, 300], [32, 20], True, 32, 8),
]


@pytest.mark.parametrize("name,ctx,ql,causal,hq,hkv", PREFILL_D256,
                         ids=[c[0] for c in PREFILL_D256])
@pytest.mark.parametrize("out_dtype,with_lse", [(torch.bfloat16, True), (torch.float32, True),
                                                (torch.bfloat16, False)],
                         ids=["bf16", "f32", "bf16_nolse"])
def test_prefill_head_dim_256(dev, name, ctx, ql, causal, hq, hkv, out_dtype, with_lse):
    """Query tiles at head dim 256: a 128-row Q-block on four wavefronts,
    each thread staging four 16-byte chunks of K and of V per key tile."""
    log(f"[prefill D=256 {name} {out_dtype} lse={with_lse}]")
    spec = workloads.small_spec(f"pf256_{name}", seed=1980 + sum(ql) + hq, contexts=ctx,
                                queries=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=256,
                                causal=causal, decode_layout=False)
    b = workloads.generate(spec, dev)
    T = sum(ql) * spec.num_q_heads
    rows = None
    if T > 8192:
        rng = np.random.default_rng(5)
        rows = np.unique(np.concatenate([rng.choice(T, 4096, replace=False), [0, T - 1]]))
    out, lse = run_prefill(b, out_dtype, with_lse=with_lse)
    compare(b, out, lse, rows=rows, label=f"prefill D=256 {name} lse={with_lse}")


@pytest.mark.parametrize("ts", [2, 5])
def test_prefill_head_dim_256_tile_splits(dev, ts):
    """Split query tiles at head dim 256, merged over a NaN-filled workspace."""
    log(f"[prefill D=256 tile splits {ts}]")
    spec = workloads.small_spec("pf256_ts", seed=1990 + ts, contexts=[2100, 1500],
                                queries=[300, 200], head_dim=256, decode_layout=False)
    b = workloads.generate(spec, dev)
    rng = np.random.default_rng(ts)
    T = 500 * spec.num_q_heads
    rows = np.unique(np.concatenate([rng.choice(T, 4096, replace=False), [0, T - 1]]))
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_prefill(b, dt, tile_splits=ts, stale_workspace=True)
        compare(b, out, lse, rows=rows, label=f"prefill D=256 ts={ts} {dt}")


def test_prefill_head_dim_256_dominant_logit_bitexact(dev):
    """Indexing at head dim 256: a dominant logit selects V[t*] exactly."""
    log("[prefill D=256 dominant logit]")
    L, q = 300, 40
    tstars = [0, 31, 32, 200, 259]
    spec = workloads.small_spec("dom256", seed=1931, contexts=[L] * len(tstars),
                                queries=[q] * len(tstars), head_dim=256, decode_layout=False)
    b = workloads.generate(spec, dev)
    P = spec.page_size
    b.q.zero_()
    b.q[:, :, 0] = 64.0
    for s, t in enumerate(tstars):
        for j in range(-(-L // P)):
            b.k_pool[int(b.block_tables[s, j]), :, :, 0] = 0.0
        b.k_pool[int(b.block_tables[s, t // P]), t % P, :, 0] = 64.0
    for dt in (torch.bfloat16, torch.float32):
        out, _ = run_prefill(b, dt, with_lse=False)
        for s, t in enumerate(tstars):
            want = b.v_pool[int(b.block_tables[s, t // P]), t % P].repeat_interleave(4, dim=0)
            got = out[s * q:(s + 1) * q]
            want = want.to(dt).expand_as(got)
            ok = (torch.equal(got.view(torch.int16), want.view(torch.int16))
                  if dt == torch.bfloat16 else torch.equal(got, want))
            assert ok, f"seq {s} t*={t} {dt}"


@pytest.mark.parametrize("shape", ["d64", "d256", "g16"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_mixed_batch_split_query_tiles(dev, shape, out_dtype):
    """A mixed batch whose single-token sequences are query tiles of their own
    (head dims 64 and 256, and G = 16 at head dim 128): the library's own
    launch splits the query tiles' key runs, and every row matches the
    oracle (bf16 output without LSE, the benchmark's launch; fp32 output
    with LSE)."""
    log(f"[mixed batch, split query tiles, {shape}, {out_dtype}]")
    kw = {"d64": dict(head_dim=64), "d256": dict(head_dim=256),
          "g16": dict(num_q_heads=64, num_kv_heads=4)}[shape]
    ctx = [9000, 17, 6100, 2500, 1, 8191, 2100, 700]
    ql = [1, 1, 1, 120, 1, 1, 64, 1]
    spec = workloads.small_spec(f"mix_{shape}", seed=2100 + 7 * len(kw) + len(shape),
                                contexts=ctx, queries=ql, decode_layout=False, **kw)
    b = workloads.generate(spec, dev)
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                         b.max_context_len, b.max_query_len, causal=True, out_dtype=out_dtype)
    tiles, _ = pa.select_tiles(pb)
    assert tiles.tile_splits > 1, tiles.as_dict()
    with_lse = out_dtype == torch.float32
    out, lse = run_prefill(b, out_dtype, with_lse=with_lse, stale_workspace=True)
    compare(b, out, lse, label=f"mixed {shape} ts={tiles.tile_splits} {out_dtype}")
