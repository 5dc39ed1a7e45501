"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (per element): fp32 outputs 2e-3; bf16 outputs
max(1e-2, h(ref) + 2^-8), where h(ref) = 2^(floor(log2 |ref|) - 8) is the
half-ulp of bf16 at the reference value (what rounding the exact result to
bf16 alone can cost) and 2^-8 the arithmetic budget of kernels that round
the softmax weights to bf16 before the P.V product; the widening starts at
|ref| >= 2, where the half-ulp (2^-7) leaves too little of 1e-2 for that
budget.  The natural-log LSE: 2e-3.  Indexing cases (dominant logit, page
permutation, NaN-poisoned stale slots) must match bit for bit.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from _util import batch_to_oracle
from paged_gqa_attention_pa_amd import pa, workloads

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 1e-2, torch.float32: 2e-3}
LSE_TOL = 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load()
    return torch.device("cuda:0")


def run_decode(b, out_dtype=torch.bfloat16, splits=None, with_lse=True, waves=None,
               workspace=None, variant=None):
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=b.q.device) if with_lse else None
    tiles = None
    if splits is not None or waves is not None or variant is not None:
        pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, b.spec.scale,
                             b.max_context_len, 1, out_dtype=out_dtype)
        tiles, _ = pa.select_tiles(pb)
        if splits is not None:
            tiles.num_splits = splits
        if waves is not None:
            tiles.waves_per_wg = waves
        if variant is not None:
            tiles.variant = variant
    out = pa.decode(b.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, b.spec.scale,
                    b.max_context_len, out_dtype=out_dtype, lse=lse, tiles=tiles,
                    workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def run_prefill(b, out_dtype=torch.bfloat16, with_lse=True, tile_splits=None,
                stale_workspace=False, splits=None, variant=None, workspace=None):
    """pa_prefill on a batch; tile_splits forces the query-tile split count,
    splits / variant the decode rows' split count and grid, stale_workspace
    fills the workspace with NaN first (pa_prefill needs no zeroed counters:
    its decode rows always use the separate merge); a given workspace is
    used as it is."""
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=b.q.device) if with_lse else None
    qsl = b.query_start_loc
    if qsl is None:
        qsl = torch.arange(b.num_seqs + 1, dtype=torch.int32, device=b.q.device)
    max_q = max(b.max_query_len, 1)
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, b.spec.scale,
                         b.max_context_len, max_q, causal=b.spec.causal, out_dtype=out_dtype)
    tiles, _ = pa.select_tiles(pb)
    if tile_splits is not None:
        tiles.tile_splits = tile_splits
    if splits is not None:
        tiles.num_splits = splits
    if variant is not None:
        tiles.variant = variant
    ws = pa.workspace_size(pb, tiles)
    if workspace is not None:
        assert workspace.numel() >= ws
    elif ws:
        workspace = torch.zeros(ws, dtype=torch.uint8, device=b.q.device)
        if stale_workspace:
            workspace.fill_(0xFF)  # every fp32 slot reads as NaN
    out = pa.prefill(b.q, qsl, b.k_pool, b.v_pool, b.block_tables, b.context_lens,
                     b.spec.scale, b.max_context_len, max_q,
                     causal=b.spec.causal, out_dtype=out_dtype, lse=lse, tiles=tiles,
                     workspace=workspace, problem=pb)
    torch.cuda.synchronize()
    return out, lse


def bf16_allowance(ref, tol=1e-2):
    """Per-element bar for bf16 outputs: max(tol, half-ulp of bf16 at |ref|
    + 2^-8).  Below |ref| = 2 this is the plain tol."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    half_ulp = np.where(a > 0, np.exp2(e - 8), 0.0)
    return np.maximum(tol, half_ulp + 2.0 ** -8)


def oracle_reference(b, rows=None):
    """The oracle's outputs and natural-log LSE for batch b (rows: a subset)."""
    return oracle.attention(batch_to_oracle(b), rows=rows)


def compare(b, out, lse, rows=None, label="", reference=None):
    """reference: oracle_reference(b, rows) computed earlier for the same
    batch and rows (several launches of one batch share it)."""
    ref, ref_lse = reference if reference is not None else oracle_reference(b, rows)
    D = b.spec.head_dim
    got = out.float().cpu().numpy().reshape(-1, D)
    got_lse = None if lse is None else lse.cpu().numpy().reshape(-1)
    if rows is not None:
        got = got[rows]
        got_lse = None if got_lse is None else got_lse[rows]
    tol = TOL[out.dtype]
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    diff = np.abs(got - ref)
    err = float(np.max(diff)) if got.size else 0.0
    log(f"{label}: rows={ref.shape[0]} max|err|={err:.3e} (tol {tol})")
    if out.dtype == torch.bfloat16:
        allowed = bf16_allowance(ref, tol)
        worst = float(np.max(diff - allowed)) if got.size else -1.0
        assert worst <= 0, f"{label}: error exceeds max(1e-2, half-ulp + 2^-8) by {worst}"
    else:
        assert err <= tol, f"{label}: max|err| {err} > {tol}"
    if got_lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(got_lse)), f"{label}: LSE finiteness differs"
        if fin.any():
            lerr = float(np.max(np.abs(got_lse[fin] - ref_lse[fin])))
            assert lerr <= LSE_TOL, f"{label}: LSE err {lerr}"
        assert np.all(got_lse[~fin] == -np.inf)
    return err


# ---------------------------------------------------------------- decode ----

DECODE_CASES = [
    ("ragged", [1, 15, 16, 17, 300, 1000, 0, 2049], 32, 8),
    ("g1", [100, 33, 257], 8, 8),
    ("g2", [100, 33, 257], 16, 8),
    ("g8", [100, 33, 257], 32, 4),
    ("g16", [100, 33, 257], 16, 1),
    ("skewed", [5000, 0, 1, 17, 3000, 0, 64, 2049, 16, 700], 32, 8),
]

MERGE_VARIANT = {"fused": 0, "separate": 2, "even": 6}


@pytest.mark.parametrize("name,ctx,hq,hkv", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
@pytest.mark.parametrize("splits", [None, 1, 3, 64])
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("merge", ["fused", "separate", "even"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_small(dev, name, ctx, hq, hkv, splits, waves, merge, out_dtype):
    log(f"[decode {name} splits={splits} waves={waves} {merge} {out_dtype}]")
    spec = workloads.small_spec(f"dec_{name}", seed=100 + len(ctx) + hq, contexts=ctx,
                                queries=[1] * len(ctx), num_q_heads=hq, num_kv_heads=hkv)
    b = workloads.generate(spec, dev)
    out, lse = run_decode(b, out_dtype, splits, waves=waves, variant=MERGE_VARIANT[merge])
    compare(b, out, lse, label=f"decode {name} S={splits} W={waves} {merge}")


def test_decode_workspace_reuse(dev):
    """One zero-filled workspace serves many calls: the merge counters reset."""
    log("[decode workspace reuse]")
    spec = workloads.small_spec("reuse", seed=9, contexts=[3000, 40, 1200], queries=[1, 1, 1])
    b = workloads.generate(spec, dev)
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                         b.max_context_len, 1)
    t, _ = pa.select_tiles(pb)
    t.num_splits = 64  # the largest split count used below
    ws = torch.zeros(pa.workspace_size(pb, t), dtype=torch.uint8, device=dev)
    first = None
    for S in (16, 16, 5, 64, 16):
        out, lse = run_decode(b, torch.float32, S, workspace=ws)
        compare(b, out, lse, label=f"reuse S={S}")
        if S == 16:
            if first is None:
                first = out.clone()
            else:
                assert torch.equal(out, first), "same call, different bits"


@pytest.mark.parametrize("splits", [2, 8, 64])
def test_decode_even_grid_stale_workspace(dev, splits):
    """Even-work grid over a workspace holding garbage (0xFF bytes: NaN
    partials, piece counts of -1) from an earlier user: every slot and count
    it reads is written by this call, or the row is empty or single-piece."""
    log(f"[decode even grid, stale workspace, S={splits}]")
    spec = workloads.small_spec("even_stale", seed=13, contexts=[4000, 0, 33, 1, 2500, 16, 0, 900],
                                queries=[1] * 8, pool_slack=20)
    b = workloads.generate(spec, dev)
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale,
                         b.max_context_len, 1, out_dtype=torch.float32)
    t, _ = pa.select_tiles(pb)
    t.num_splits, t.variant = splits, 6
    ws = torch.full((pa.workspace_size(pb, t),), 0xFF, dtype=torch.uint8, device=dev)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=dev)
    out = pa.decode(b.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, spec.scale,
                    b.max_context_len, out_dtype=torch.float32, lse=lse, tiles=t, workspace=ws,
                    problem=pb)
    torch.cuda.synchronize()
    compare(b, out, lse, label=f"even stale S={splits}")


def test_decode_logit_stress(dev):
    log("[decode logit x8 stress]")
    spec = workloads.small_spec("dec_stress", seed=7, contexts=[5000, 123], queries=[1, 1],
                                logit_gain=8.0)
    b = workloads.generate(spec, dev)
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_decode(b, dt)
        compare(b, out, lse, label=f"decode stress {dt}")


def _dominant_batch(dev, tstars, L, prefill_q=None):
    qlen = [1] if prefill_q is None else [prefill_q]
    spec = workloads.small_spec("dom", seed=31, contexts=[L] * len(tstars),
                                queries=qlen * len(tstars))
    b = workloads.generate(spec, dev)
    P = spec.page_size
    # q = 64 e_0 on every head; k_t*[0] = 64 on every KV head, k_t[0] = 0 elsewhere:
    # z_t* = 4096 * scale ~ 362 and z_t = 0, so every other weight is exp(-362) -> 0.
    b.q.zero_()
    b.q[:, :, 0] = 64.0
    for s, t in enumerate(tstars):
        n = -(-L // P)
        for j in range(n):
            page = int(b.block_tables[s, j])
            b.k_pool[page, :, :, 0] = 0.0
        page = int(b.block_tables[s, t // P])
        b.k_pool[page, t % P, :, 0] = 64.0
    return b


@pytest.mark.parametrize("splits", [1, 5, 64])
def test_decode_dominant_logit_bitexact(dev, splits):
    log(f"[decode dominant logit S={splits}]")
    L = 1000
    tstars = [0, 15, 16, 500, 511, 999]
    b = _dominant_batch(dev, tstars, L)
    for dt in (torch.bfloat16, torch.float32):
        out, _ = run_decode(b, dt, splits)
        for s, t in enumerate(tstars):
            page = int(b.block_tables[s, t // 16])
            v = b.v_pool[page, t % 16]  # [Hkv, D]
            want = v.repeat_interleave(4, dim=0).to(dt)
            assert torch.equal(out[s].view(torch.int16) if dt == torch.bfloat16 else out[s],
                               want.view(torch.int16) if dt == torch.bfloat16 else want), \
                f"seq {s} t*={t} {dt}"


def _permuted(b):
    """Same problem with every page moved elsewhere and the tables remapped."""
    g = torch.Generator(device="cpu")
    g.manual_seed(77)
    npool = b.k_pool.shape[0]
    perm = torch.randperm(npool, generator=g).to(b.k_pool.device)
    k2 = torch.empty_like(b.k_pool)
    v2 = torch.empty_like(b.v_pool)
    k2[perm] = b.k_pool
    v2[perm] = b.v_pool
    bt2 = torch.where(b.block_tables >= 0, perm[b.block_tables.clamp(min=0).long()].int(),
                      b.block_tables)
    return workloads.Batch(spec=b.spec, q=b.q, k_pool=k2, v_pool=v2, block_tables=bt2,
                           context_lens=b.context_lens, query_start_loc=b.query_start_loc,
                           query_lens=b.query_lens, used_pages=b.used_pages)


def test_decode_page_permutation_and_nan_bitexact(dev):
    log("[decode permutation / NaN poison]")
    spec = workloads.small_spec("perm", seed=41, contexts=[37, 1000, 16, 513], queries=[1] * 4,
                                pool_slack=40)
    b = workloads.generate(spec, dev, fill="nan")
    bz = workloads.generate(spec, dev, fill="zero")
    for splits in (1, 7):
        o1, l1 = run_decode(b, torch.float32, splits)
        o2, l2 = run_decode(_permuted(b), torch.float32, splits)
        o3, l3 = run_decode(bz, torch.float32, splits)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert torch.equal(o1, o3) and torch.equal(l1, l3)
        assert torch.isfinite(o1).all()


# ---------------------------------------------------------------- prefill ---

PREFILL_CASES = [
    # (name, contexts, query lens, causal)
    ("chunks", [300, 77, 1000, 33], [140, 77, 31, 33], True),
    ("tiles", [32, 64, 65, 200], [32, 64, 65, 129], True),
    ("noncausal", [300, 50], [100, 7], False),
    ("decode_rows_first", [900, 40, 260, 513], [1, 1, 100, 200], True),
    ("decode_rows_last", [260, 513, 900, 40], [100, 200, 1, 1], True),
    ("degenerate", [0, 1, 5, 16], [0, 1, 5, 1], True),
    # more than 2048 16-key blocks: the LDS window of block offsets is
    # restaged mid-sequence
    ("long_context", [40000, 300], [32, 20], True),
    ("long_noncausal", [34000], [40], False),
]


@pytest.mark.parametrize("name,ctx,ql,causal", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
@pytest.mark.parametrize("out_dtype,with_lse", [(torch.bfloat16, True), (torch.float32, True),
                                                (torch.bfloat16, False)],
                         ids=["bf16", "f32", "bf16_nolse"])
def test_prefill_small(dev, name, ctx, ql, causal, out_dtype, with_lse):
    """bf16 output without an LSE is the launch the benchmark times: P
    rounded to bf16, one P.V MFMA per step (the others carry P as bf16 high
    part + remainder)."""
    log(f"[prefill {name} {out_dtype} lse={with_lse}]")
    spec = workloads.small_spec(f"pre_{name}", seed=200 + sum(ql), contexts=ctx, queries=ql,
                                causal=causal, decode_layout=False)
    b = workloads.generate(spec, dev)
    out, lse = run_prefill(b, out_dtype, with_lse=with_lse)
    compare(b, out, lse, label=f"prefill {name} lse={with_lse}")


MIXED_EVEN_CASES = [
    # (name, contexts, query lens): single-token sequences after, before and
    # between prefill chunks, an empty context among them
    ("decodes_last", [260, 513, 900, 40], [100, 200, 1, 1]),
    ("decodes_first", [900, 40, 260, 513], [1, 1, 100, 200]),
    ("interleaved", [2000, 300, 700, 1, 5000, 0], [1, 150, 1, 1, 64, 1]),
]


@pytest.mark.parametrize("name,ctx,ql", MIXED_EVEN_CASES, ids=[c[0] for c in MIXED_EVEN_CASES])
@pytest.mark.parametrize("splits", [2, 8, 33])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_mixed_even_grid(dev, name, ctx, ql, splits, out_dtype):
    """A mixed batch whose decode rows run on the even-work grid (variant
    bits 1 and 2) with several splits, over a zero-filled workspace, every
    row compared: the merge must read the decode rows' partials where the
    decode workgroups wrote them (sequence rows) and leave prefill rows
    alone."""
    log(f"[mixed even grid {name} S={splits} {out_dtype}]")
    spec = workloads.small_spec(f"mixeven_{name}", seed=900 + splits + sum(ql), contexts=ctx,
                                queries=ql, decode_layout=False)
    b = workloads.generate(spec, dev)
    variant = 6 | (1 if out_dtype == torch.float32 else 0)
    out, lse = run_prefill(b, out_dtype, splits=splits, variant=variant)
    compare(b, out, lse, label=f"mixed even {name} S={splits}")


@pytest.mark.parametrize("splits", [4, 33])
def test_mixed_after_decode_same_workspace(dev, splits):
    """A decode-only call and then a mixed call share one workspace: the
    piece counts the decode call left for units that are prefill chunks in
    the mixed call must not reach the mixed call's output."""
    log(f"[mixed after decode, shared workspace, S={splits}]")
    dspec = workloads.small_spec("shared_dec", seed=950 + splits, contexts=[3000, 4000, 900, 40],
                                 queries=[1, 1, 1, 1], decode_layout=False)
    mspec = workloads.small_spec("shared_mix", seed=960 + splits, contexts=[260, 513, 900, 40],
                                 queries=[100, 200, 1, 1], decode_layout=False)
    bd = workloads.generate(dspec, dev)
    bm = workloads.generate(mspec, dev)
    sizes = []
    for b in (bd, bm):
        pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, b.spec.scale,
                             b.max_context_len, max(b.max_query_len, 1), out_dtype=torch.float32)
        t, _ = pa.select_tiles(pb)
        t.num_splits, t.variant = splits, 7
        sizes.append(pa.workspace_size(pb, t))
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device=dev)
    out_d, lse_d = run_prefill(bd, torch.float32, splits=splits, variant=7, workspace=ws)
    compare(bd, out_d, lse_d, label=f"shared ws decode S={splits}")
    out_m, lse_m = run_prefill(bm, torch.float32, splits=splits, variant=7, workspace=ws)
    compare(bm, out_m, lse_m, label=f"shared ws mixed S={splits}")


TILE_SPLIT_CASES = [
    # (name, contexts, query lens, causal): runs long enough to split, runs of
    # one tile or none, decode rows beside split tiles, no causal mask
    ("long_prefix", [2100, 1500], [300, 200], True),
    ("short_runs", [40, 64, 65, 200], [40, 64, 65, 129], True),
    ("decode_rows_first", [900, 40, 2600, 513], [1, 1, 100, 200], True),
    ("noncausal", [3000, 50], [100, 7], False),
]


@pytest.mark.parametrize("name,ctx,ql,causal", TILE_SPLIT_CASES,
                         ids=[c[0] for c in TILE_SPLIT_CASES])
@pytest.mark.parametrize("ts", [2, 3, 8])
def test_prefill_tile_splits(dev, name, ctx, ql, causal, ts):
    """Query tiles whose keys are cut into ts runs, merged by log-sum-exp,
    over a NaN-filled workspace, in both output precisions."""
    log(f"[prefill tile splits {name} ts={ts}]")
    spec = workloads.small_spec(f"pts_{name}", seed=700 + ts + sum(ql), contexts=ctx,
                                queries=ql, causal=causal, decode_layout=False)
    b = workloads.generate(spec, dev)
    T = sum(ql) * spec.num_q_heads
    rows = None
    if T > 4096:  # sample rows, always including the first and last of each sequence
        rng = np.random.default_rng(ts)
        rows = np.unique(np.concatenate([rng.choice(T, 2048, replace=False),
                                         np.array([0, T - 1])]))
    for dt in (torch.bfloat16, torch.float32):
        out, lse = run_prefill(b, dt, tile_splits=ts, stale_workspace=True)
        compare(b, out, lse, rows=rows, label=f"tile splits {name} ts={ts} {dt}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 4), (16, 1)])
def test_prefill_group_sizes(dev, hq, hkv):
    log(f"[prefill G={hq // hkv}]")
    spec = workloads.small_spec("pre_g", seed=300 + hq + hkv, contexts=[200, 90], queries=[70, 90],
                                num_q_heads=hq, num_kv_heads=hkv, decode_layout=False)
    b = workloads.generate(spec, dev)
    out, lse = run_prefill(b, torch.float32)
    compare(b, out, lse, label=f"prefill G={hq // hkv}")


def test_prefill_dominant_logit_bitexact(dev):
    log("[prefill dominant logit]")
    L, q = 300, 40
    tstars = [0, 31, 32, 200, 259]  # all <= L - q, so every row of the chunk sees t*
    b = _dominant_batch(dev, tstars, L, prefill_q=q)
    for dt, ts in ((torch.bfloat16, 1), (torch.float32, 1), (torch.bfloat16, 3),
                   (torch.float32, 8)):
        out, _ = run_prefill(b, dt, tile_splits=ts)
        for s, t in enumerate(tstars):
            page = int(b.block_tables[s, t // 16])
            want = b.v_pool[page, t % 16].repeat_interleave(4, dim=0).to(dt)
            got = out[s * q:(s + 1) * q]
            ok = (torch.equal(got.view(torch.int16), want.view(torch.int16).expand_as(got))
                  if dt == torch.bfloat16 else torch.equal(got, want.expand_as(got)))
            assert ok, f"seq {s} t*={t} {dt} tile_splits={ts}"


def test_prefill_page_permutation_and_nan_bitexact(dev):
    log("[prefill permutation / NaN poison]")
    spec = workloads.small_spec("pperm", seed=43, contexts=[301, 77, 40], queries=[150, 77, 1],
                                pool_slack=30, decode_layout=False)
    b = workloads.generate(spec, dev, fill="nan")
    bz = workloads.generate(spec, dev, fill="zero")
    o1, l1 = run_prefill(b, torch.float32)
    o2, l2 = run_prefill(_permuted(b), torch.float32)
    o3, l3 = run_prefill(bz, torch.float32)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    # the same with split query tiles (and stale partial slots)
    s1, m1 = run_prefill(b, torch.float32, tile_splits=3, stale_workspace=True)
    s2, m2 = run_prefill(_permuted(b), torch.float32, tile_splits=3, stale_workspace=True)
    s3, m3 = run_prefill(bz, torch.float32, tile_splits=3)
    assert torch.equal(s1, s2) and torch.equal(m1, m2)
    assert torch.equal(s1, s3) and torch.equal(m1, m3)


# ---------------------------------------------------------------- reduce ----

@pytest.mark.parametrize("S,D", [(1, 128), (2, 128), (7, 128), (64, 128), (256, 128),
                                 (1000, 64), (4096, 128), (33, 256), (3, 1024), (17, 12),
                                 (5, 4)])
def test_reduce_random_partials(dev, S, D):
    """pa_splitkv_reduce alone over its whole argument range: 1 to 4096
    splits, head dims from 4 to 1024 (any multiple of 4)."""
    log(f"[reduce S={S} D={D}]")
    g = torch.Generator(device="cpu")
    g.manual_seed(500 + S + D)
    rows = 37
    po = torch.randn((rows, S, D), generator=g, dtype=torch.float32)
    pl = torch.randn((rows, S), generator=g, dtype=torch.float32) * 20
    drop = torch.rand((rows, S), generator=g) < 0.3
    pl[drop] = -math.inf
    pl[3] = -math.inf  # a row with every split empty
    ref, ref_lse = oracle.merge(po.double().numpy(), pl.double().numpy())
    for dt in (torch.float32, torch.bfloat16):
        lse = torch.empty(rows, dtype=torch.float32, device=dev)
        out = pa.splitkv_reduce(po.to(dev), pl.to(dev), out_dtype=dt, lse=lse)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        tol = 2e-3 if dt == torch.float32 else 2e-2  # |O| reaches ~4 here
        assert np.max(np.abs(got - ref)) <= tol
        gl = lse.cpu().numpy()
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(gl))
        assert np.max(np.abs(gl[fin] - ref_lse[fin])) <= LSE_TOL
        assert np.all(got[3] == 0)


# ------------------------------------------------------- named workloads ----

def _sample_rows(b, n, seed):
    T, Hq = b.q.shape[:2]
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T * Hq, size=min(n, T * Hq), replace=False).tolist())
    # always include the first and last token of every sequence, all heads
    if b.query_start_loc is not None:
        qsl = b.query_start_loc.cpu().tolist()
        for s in range(b.num_seqs):
            for t in {qsl[s], qsl[s + 1] - 1}:
                if qsl[s + 1] > qsl[s]:
                    rows.update(t * Hq + h for h in range(Hq))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("layout", workloads.KV_LAYOUTS)
@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER + ["decode_b256_ctx8k"])
def test_named_workload(dev, name, layout):
    """Each workload at full size, launched as the benchmark launches it
    (table launch shape, bf16 output, no LSE: for the query-tile and
    short-run kernels that is the variant with P rounded to bf16), with the
    pools' pages stored in either order (the benchmark stores them head
    major), every row compared with the oracle except at batch 256 (a
    seeded sample); query-layout workloads are also run with an LSE (the
    precise variant) on sampled rows."""
    log(f"[workload {name} {layout}]")
    spec = workloads.WORKLOADS[name]
    b = workloads.with_layout(workloads.generate(spec, dev, fill="nan"), layout)
    if spec.decode_layout:
        out, _ = run_decode(b, torch.bfloat16, with_lse=False)
        rows = None
        if b.num_seqs > 64:  # 8192 rows of 8192 keys: a seeded sample, the first and last rows
            rng = np.random.default_rng(3)
            n = b.num_seqs * spec.num_q_heads
            rows = np.union1d(rng.choice(n, 480, replace=False), [0, 1, n - 2, n - 1])
        compare(b, out, None, rows=rows, label=f"workload {name}")
        out, lse = run_decode(b, torch.bfloat16)
        compare(b, out, lse, rows=rows, label=f"workload {name} with lse")
    else:
        out, _ = run_prefill(b, torch.bfloat16, with_lse=False)
        compare(b, out, None, label=f"workload {name} (benchmarked launch, all rows)")
        del out
        out, lse = run_prefill(b, torch.bfloat16)
        rows = _sample_rows(b, 3000, seed=1)
        if name == "mixed_unified":  # every decode row too
            dec = np.arange(16 * 32, dtype=np.int64)
            rows = np.union1d(rows, dec)
        compare(b, out, lse, rows=rows, label=f"workload {name} with lse")
    if name == "decode_ctx512":
        out32, lse32 = run_decode(b, torch.float32)
        compare(b, out32, lse32, label="workload decode_ctx512 fp32")
