"""GPU parity at page sizes above 16 (P = 32, 64, 256) against the fp64 oracle.

A page of P = 16 * 2^k slots is 2^k consecutive 16-key tiles: the kernels
look block-table entry t >> k up for tile t and start 16 * (t mod 2^k) slots
into that page.  Each test below runs one path at these page sizes: decode
on its three grids, short query runs, query tiles at head dims 64, 128 and
256 (with split tiles and the page window restaged), mixed batches, the
paged append and the input checks.  A re-paging test moves one batch's
K and V into pages of another size and expects every output bit unchanged,
since no kernel's arithmetic order depends on where a key sits.
"""
import dataclasses

import numpy as np
import pytest
import torch

from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_append import append_and_check
from test_gpu_parity import MERGE_VARIANT, compare, dev, log, run_decode, run_prefill  # noqa: F401

pytestmark = pytest.mark.gpu

PAGES = [32, 64, 256]
DECODE_CTX = [1, 15, 16, 17, 31, 32, 33, 300, 1000, 0, 2049, 5000]


@pytest.mark.parametrize("P", PAGES)
@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8), (16, 1)], ids=["g4", "g8", "g16"])
@pytest.mark.parametrize("splits", [None, 3])
@pytest.mark.parametrize("merge", ["fused", "separate", "even"])
def test_decode_page_size(dev, P, hq, hkv, splits, merge):
    log(f"[decode P={P} G={hq // hkv} S={splits} {merge}]")
    spec = workloads.small_spec(f"dec_p{P}", seed=3000 + P + hq, contexts=DECODE_CTX,
                                queries=[1] * len(DECODE_CTX), num_q_heads=hq,
                                num_kv_heads=hkv, page_size=P)
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_decode(b, dt, splits, variant=MERGE_VARIANT[merge])
        compare(b, out, lse, label=f"decode P={P} G={hq // hkv} S={splits} {merge} {dt}")


@pytest.mark.parametrize("P", PAGES)
@pytest.mark.parametrize("waves", [4, 8])
def test_decode_page_size_waves(dev, P, waves):
    log(f"[decode P={P} waves={waves}]")
    spec = workloads.small_spec(f"decw_p{P}", seed=3100 + P + waves, contexts=DECODE_CTX,
                                queries=[1] * len(DECODE_CTX), page_size=P)
    b = workloads.generate(spec, dev)
    for splits in (1, 64):
        out, lse = run_decode(b, torch.float32, splits, waves=waves)
        compare(b, out, lse, label=f"decode P={P} W={waves} S={splits}")


SHORT_RUNS = [
    # (name, contexts, query lens, causal)
    ("q2", [64, 2049, 33, 700, 8, 1, 16], [2, 2, 2, 2, 2, 1, 2], True),
    ("q4_ragged", [5, 300, 1000, 4100, 0], [4, 3, 4, 1, 0], True),
    ("noncausal", [300, 45, 1000], [6, 4, 8], False),
]


@pytest.mark.parametrize("P", PAGES)
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("name,ctx,ql,causal", SHORT_RUNS, ids=[c[0] for c in SHORT_RUNS])
def test_short_runs_page_size(dev, P, d, name, ctx, ql, causal):
    log(f"[short runs P={P} D={d} {name}]")
    spec = workloads.small_spec(f"sr_p{P}_{name}", seed=3200 + P + d + sum(ql), contexts=ctx,
                                queries=ql, head_dim=d, causal=causal, decode_layout=False,
                                page_size=P)
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_prefill(b, dt)
        compare(b, out, lse, label=f"short runs P={P} D={d} {name} {dt}")


PREFILL = [
    # (name, contexts, query lens, causal)
    ("chunks", [300, 77, 1000, 33], [140, 77, 31, 33], True),
    ("tiles", [32, 64, 65, 200], [32, 64, 65, 129], True),
    ("noncausal", [300, 50], [100, 7], False),
    ("decode_rows", [900, 40, 260, 513], [1, 1, 100, 200], True),
    # past the page window (32k keys at head dims 64 and 128, 16k at 256):
    # the window is restaged mid-sequence, its blocks spread over pages
    ("long_context", [40000, 300], [32, 20], True),
]


def _rows(T, seed, n=4096):
    if T <= 8192:
        return None
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.choice(T, n, replace=False), [0, T - 1]]))


@pytest.mark.parametrize("P", PAGES)
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("name,ctx,ql,causal", PREFILL, ids=[c[0] for c in PREFILL])
def test_prefill_page_size(dev, P, d, name, ctx, ql, causal):
    log(f"[prefill P={P} D={d} {name}]")
    spec = workloads.small_spec(f"pf_p{P}_{name}", seed=3300 + P + d + sum(ql), contexts=ctx,
                                queries=ql, head_dim=d, causal=causal, decode_layout=False,
                                page_size=P)
    b = workloads.generate(spec, dev)
    rows = _rows(sum(ql) * spec.num_q_heads, P + d)
    for dt, with_lse in ((torch.bfloat16, False), (torch.float32, True)):
        out, lse = run_prefill(b, dt, with_lse=with_lse)
        compare(b, out, lse, rows=rows, label=f"prefill P={P} D={d} {name} {dt}")


@pytest.mark.parametrize("P", PAGES)
@pytest.mark.parametrize("d", [64, 128, 256])
def test_prefill_page_size_tile_splits(dev, P, d):
    log(f"[prefill P={P} D={d} tile splits]")
    spec = workloads.small_spec(f"pfts_p{P}", seed=3400 + P + d, contexts=[2100, 1500],
                                queries=[300, 200], head_dim=d, decode_layout=False,
                                page_size=P)
    b = workloads.generate(spec, dev)
    rows = _rows(500 * spec.num_q_heads, P + d + 1)
    for ts in (2, 5):
        out, lse = run_prefill(b, torch.float32, tile_splits=ts, stale_workspace=True)
        compare(b, out, lse, rows=rows, label=f"prefill P={P} D={d} ts={ts}")


@pytest.mark.parametrize("P", PAGES)
@pytest.mark.parametrize("splits", [2, 33])
def test_mixed_even_grid_page_size(dev, P, splits):
    """Decode rows on the even-work grid beside query tiles, every row compared."""
    log(f"[mixed even grid P={P} S={splits}]")
    ctx, ql = [2000, 300, 700, 1, 5000, 0], [1, 150, 1, 1, 64, 1]
    spec = workloads.small_spec(f"mix_p{P}", seed=3500 + P + splits, contexts=ctx, queries=ql,
                                decode_layout=False, page_size=P)
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        variant = 6 | (1 if dt == torch.float32 else 0)
        out, lse = run_prefill(b, dt, splits=splits, variant=variant)
        compare(b, out, lse, label=f"mixed even P={P} S={splits} {dt}")


def _dominant(dev, P, tstars, L, q):
    spec = workloads.small_spec(f"dom_p{P}", seed=3600 + P, contexts=[L] * len(tstars),
                                queries=[q] * len(tstars), page_size=P,
                                decode_layout=(q == 1))
    b = workloads.generate(spec, dev)
    # q = 64 e_0 on every head and k_t*[0] = 64, k_t[0] = 0 elsewhere: every
    # other weight is exp(-362) -> 0, so the output row is V[t*] exactly
    b.q.zero_()
    b.q[:, :, 0] = 64.0
    for s, t in enumerate(tstars):
        for j in range(-(-L // P)):
            b.k_pool[int(b.block_tables[s, j]), :, :, 0] = 0.0
        b.k_pool[int(b.block_tables[s, t // P]), t % P, :, 0] = 64.0
    return b


@pytest.mark.parametrize("P", PAGES)
def test_dominant_logit_bitexact_page_size(dev, P):
    """Slot indexing inside large pages: a dominant logit at key t* selects
    V[t*] bit for bit, for t* on either side of 16-key tile and page edges."""
    log(f"[dominant logit P={P}]")
    L = 1000
    tstars = sorted({0, 15, 16, P - 1, P, P + 17, 2 * P - 1, 500, 959})
    tstars = [t for t in tstars if t < L]
    for q in (1, 40):
        b = _dominant(dev, P, tstars, L, q)
        for dt in (torch.bfloat16, torch.float32):
            if q == 1:
                out, _ = run_decode(b, dt, 5)
            else:
                out, _ = run_prefill(b, dt, with_lse=False)
            for s, t in enumerate(tstars):
                want = b.v_pool[int(b.block_tables[s, t // P]), t % P]
                want = want.repeat_interleave(4, dim=0).to(dt)
                got = out[s * q:(s + 1) * q]
                ok = (torch.equal(got.view(torch.int16), want.view(torch.int16).expand_as(got))
                      if dt == torch.bfloat16 else torch.equal(got, want.expand_as(got)))
                assert ok, f"P={P} q={q} seq {s} t*={t} {dt}"


def _repaged(b, P, seed):
    """The same keys and values in pages of P slots, pages in random order,
    every slot no context covers NaN."""
    spec = b.spec
    ctx = [int(c) for c in b.context_lens.cpu()]
    need = [-(-c // P) for c in ctx]
    npool = sum(need) + 5
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    perm = torch.randperm(npool, generator=g)
    Hkv, D, P0 = spec.num_kv_heads, spec.head_dim, spec.page_size
    pools = [torch.full((npool, P, Hkv, D), float("nan"), dtype=torch.bfloat16, device=b.q.device)
             for _ in range(2)]
    bt = torch.full((len(ctx), max(max(need), 1)), -1, dtype=torch.int32)
    off = 0
    for s, L in enumerate(ctx):
        bt[s, :need[s]] = perm[off:off + need[s]].to(torch.int32)
        off += need[s]
        for src, dst in ((b.k_pool, pools[0]), (b.v_pool, pools[1])):
            pages = b.block_tables[s, :-(-L // P0)].long()
            dense = src[pages].reshape(-1, Hkv, D)[:L]
            for j in range(need[s]):
                rows = dense[j * P:(j + 1) * P]
                dst[int(bt[s, j]), :rows.shape[0]] = rows
    bspec = dataclasses.replace(spec, page_size=P, pool_pages=npool, max_blocks=None)
    return workloads.Batch(spec=bspec, q=b.q, k_pool=pools[0], v_pool=pools[1],
                           block_tables=bt.to(b.q.device), context_lens=b.context_lens,
                           query_start_loc=b.query_start_loc, query_lens=b.query_lens,
                           used_pages=None)


@pytest.mark.parametrize("P", PAGES)
def test_repaging_is_bitexact(dev, P):
    """One batch in 16-slot pages and again in P-slot pages: identical bits
    from decode (both grids) and from query tiles, split or not."""
    log(f"[re-paging 16 -> {P}]")
    dspec = workloads.small_spec("rp_dec", seed=3700, contexts=DECODE_CTX,
                                 queries=[1] * len(DECODE_CTX))
    b16 = workloads.generate(dspec, dev)
    bP = _repaged(b16, P, seed=P)
    for merge in ("fused", "even"):
        for splits in (1, 7):
            o1, l1 = run_decode(b16, torch.float32, splits, variant=MERGE_VARIANT[merge])
            o2, l2 = run_decode(bP, torch.float32, splits, variant=MERGE_VARIANT[merge])
            assert torch.equal(o1, o2) and torch.equal(l1, l2), f"decode {merge} S={splits}"
    pspec = workloads.small_spec("rp_pre", seed=3701, contexts=[300, 77, 1000, 40, 2100],
                                 queries=[140, 77, 31, 1, 3], decode_layout=False)
    b16 = workloads.generate(pspec, dev)
    bP = _repaged(b16, P, seed=P + 1)
    for ts in (None, 3):
        o1, l1 = run_prefill(b16, torch.float32, tile_splits=ts)
        o2, l2 = run_prefill(bP, torch.float32, tile_splits=ts)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"prefill ts={ts}"


@pytest.mark.parametrize("P", PAGES)
def test_append_page_size(dev, P):
    log(f"[append P={P}]")
    spec = workloads.small_spec(f"app_p{P}", seed=3800 + P, contexts=[1, 15, 300, 1000, 33, P],
                                queries=[1, 15, 100, 1, 16, P], page_size=P, pool_slack=9)
    b = workloads.generate(spec, dev)
    kn, vn = workloads.new_kv(b, seed=3810 + P)
    append_and_check(b, kn, vn, f"append P={P}")


@pytest.mark.parametrize("P", PAGES)
def test_check_inputs_page_size(dev, P):
    """Block counts per context follow the page size: ceil(L / P) entries
    are checked, and a context one slot past its row is reported."""
    log(f"[check inputs P={P}]")
    spec = workloads.small_spec(f"chk_p{P}", seed=3900 + P, contexts=[700, 33, 1, 5, 2049],
                                queries=[1] * 5, page_size=P)
    b = workloads.generate(spec, dev)
    pages = b.k_pool.shape[0]

    def flags(bt=None, ctx=None, max_ctx=None):
        bt = b.block_tables if bt is None else bt
        ctx = b.context_lens if ctx is None else ctx
        pb = pa.make_problem(b.q, b.k_pool, bt, b.num_seqs, b.spec.scale,
                             b.max_context_len if max_ctx is None else max_ctx, 1)
        return pa.check_inputs(pb, pages, bt, ctx, None)

    assert flags() == 0
    # the last entry a context uses is checked, the one after it is not
    L0 = int(b.context_lens[0])
    n0 = -(-L0 // P)
    bt = b.block_tables.clone()
    bt[0, n0 - 1] = pages
    assert flags(bt=bt) == pa.CHECK_PAGE
    if n0 < bt.shape[1]:
        bt = b.block_tables.clone()
        bt[0, n0:] = pages + 3
        assert flags(bt=bt) == 0
    rows = b.block_tables.shape[1]
    ctx = b.context_lens.clone()
    ctx[1] = rows * P + 1
    bt = b.block_tables.clone()
    bt[1, :] = 0
    assert flags(bt=bt, ctx=ctx, max_ctx=rows * P) == (pa.CHECK_CONTEXT_BLOCKS |
                                                        pa.CHECK_CONTEXT_BOUND)


def test_largest_page_size(dev):
    """Pages of 1024 slots (64 tiles each): decode on both grids, a short
    run and query tiles, with contexts inside the first page, across pages
    and ending one slot into a page."""
    P = 1024
    log("[page size 1024]")
    ctx = [1, 1000, 1025, 3000, 0, 4097]
    spec = workloads.small_spec("p1024_dec", seed=3950, contexts=ctx, queries=[1] * len(ctx),
                                page_size=P)
    b = workloads.generate(spec, dev)
    for merge in ("separate", "even"):
        out, lse = run_decode(b, torch.float32, 5, variant=MERGE_VARIANT[merge])
        compare(b, out, lse, label=f"decode P={P} {merge}")
    spec = workloads.small_spec("p1024_pre", seed=3951, contexts=[3000, 1025, 40, 4097],
                                queries=[300, 4, 40, 1], page_size=P, decode_layout=False)
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_prefill(b, dt)
        compare(b, out, lse, label=f"prefill P={P} {dt}")
    spec = workloads.small_spec("p1024_sr", seed=3952, contexts=[3000, 1025, 40, 4097],
                                queries=[4, 3, 4, 2], page_size=P, decode_layout=False)
    b = workloads.generate(spec, dev)
    out, lse = run_prefill(b, torch.float32)
    compare(b, out, lse, label=f"short runs P={P}")
