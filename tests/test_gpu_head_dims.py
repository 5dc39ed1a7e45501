"""GPU parity at head dims 64 and 256 against the fp64 oracle.

Decode and short query runs at these head dims run on the short-run kernel
(one Q-block per (sequence, kv head) unit, MFMA for both products); the
paged append copies rows of any head dim bit for bit.  Longer query runs
take the query-tile kernel, built for head dims 64 and 128: at 256
pa_prefill reports them as unsupported.
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


def test_long_runs_unsupported_d256(dev):
    spec = workloads.small_spec("long_d256", seed=970, contexts=[300], queries=[100],
                                head_dim=256, decode_layout=False)
    b = workloads.generate(spec, dev)
    with pytest.raises(pa.PAError) as e:
        run_prefill(b, torch.bfloat16)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED
