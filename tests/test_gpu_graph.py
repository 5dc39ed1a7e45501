"""HIP-graph capture and replay (the static launch grid + graphs steps of the
IBM Triton summary's five-step list): a decode step and a mixed prefill step
are captured once; lengths, block tables and queries are then rewritten in
place (within the capture-time bounds) and every replay is checked against
the oracle.  Eager work and synchronisations run between replays, and a
repeated replay must reproduce the same bits.  Also captured: the even-work
decode grid (with 64-slot pages), the short-run path, and the allocation-free
decode entry point."""
import numpy as np
import pytest
import torch

from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_parity import compare, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load()
    return torch.device("cuda:0")


def _refill(b, contexts, seed, dev):
    """Same tensors, new lengths / tables / queries (pages stay in the pool)."""
    P = b.spec.page_size
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    perm = torch.randperm(b.k_pool.shape[0], generator=g)
    bt = torch.full(tuple(b.block_tables.shape), -1, dtype=torch.int32)
    off = 0
    for s, L in enumerate(contexts):
        n = -(-L // P)
        bt[s, :n] = perm[off:off + n].to(torch.int32)
        off += n
    b.block_tables.copy_(bt.to(dev))
    b.context_lens.copy_(torch.tensor(contexts, dtype=torch.int32).to(dev))
    b.q.copy_(torch.randn(tuple(b.q.shape), generator=g).to(torch.bfloat16).to(dev))
    # pages the new tables use must hold finite data: draw them fresh
    used = perm[:off].to(dev)
    shape = (off,) + tuple(b.k_pool.shape[1:])
    b.k_pool[used] = torch.randn(shape, generator=g).to(torch.bfloat16).to(dev)
    b.v_pool[used] = torch.randn(shape, generator=g).to(torch.bfloat16).to(dev)


def test_decode_graph_replay(dev):
    log("[graph decode]")
    bound = 3000
    spec = workloads.small_spec("gdec", seed=61, contexts=[bound, 700, 1500], queries=[1, 1, 1],
                                pool_slack=200)
    b = workloads.generate(spec, dev, fill="zero")
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale, bound, 1,
                         out_dtype=torch.float32)
    tiles, ws = pa.select_tiles(pb)
    tiles.num_splits = 8
    ws = pa.workspace_size(pb, tiles)
    workspace = torch.zeros(ws, dtype=torch.uint8, device=dev)
    out = torch.empty(b.q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=dev)

    def step():
        pa.decode(b.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, spec.scale, bound,
                  out=out, lse=lse, tiles=tiles, workspace=workspace, problem=pb)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rnd, ctx in enumerate([[3000, 700, 1500], [17, 2999, 1], [0, 1024, 3000]]):
        if rnd:
            _refill(b, ctx, seed=100 + rnd, dev=dev)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare(b, out, lse, label=f"graph decode replay {rnd}")
        first = out.clone()
        _ = (b.q.float() * 2).sum().item()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, first), "replay not bit-deterministic"


def test_mixed_prefill_graph_replay(dev):
    log("[graph mixed prefill]")
    bound = 1200
    ql = [1, 1, 200, 150]
    spec = workloads.small_spec("gmix", seed=62, contexts=[1200, 333, 900, 150], queries=ql,
                                pool_slack=150, decode_layout=False)
    b = workloads.generate(spec, dev, fill="zero")
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale, bound,
                         max(ql), causal=True)
    tiles, ws = pa.select_tiles(pb)
    workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
    out = torch.empty(b.q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=dev)

    def step():
        pa.prefill(b.q, b.query_start_loc, b.k_pool, b.v_pool, b.block_tables, b.context_lens,
                   spec.scale, bound, max(ql), causal=True, out=out, lse=lse, tiles=tiles,
                   workspace=workspace, problem=pb)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    # query lengths are fixed by the captured query_start_loc; contexts vary
    for rnd, ctx in enumerate([[1200, 333, 900, 150], [5, 1200, 201, 1100], [1, 1, 1200, 150]]):
        if rnd:
            _refill(b, ctx, seed=200 + rnd, dev=dev)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare(b, out, lse, label=f"graph mixed replay {rnd}")
        first = out.clone()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, first), "replay not bit-deterministic"


def _replay_rounds(b, g, out, lse, contexts, seed, label):
    """Rewrite lengths / tables / queries, replay, compare; replay again
    after unrelated eager work and expect the same bits."""
    for rnd, ctx in enumerate(contexts):
        if rnd:
            _refill(b, ctx, seed=seed + rnd, dev=b.q.device)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare(b, out, lse, label=f"{label} replay {rnd}")
        first = out.clone()
        _ = (b.q.float() * 3).sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, first), f"{label}: replay not bit-deterministic"


def test_even_grid_decode_graph_replay_pages_of_64(dev):
    """The even-work grid (every workgroup finds its share from the device
    lengths at run time) under capture, with 64-slot pages: the captured
    grid stays valid as the length mix changes under the same bounds."""
    log("[graph even-grid decode, P = 64]")
    bound = 4000
    ctx0 = [bound, 700, 1500, 64, 2200, 1]
    spec = workloads.small_spec("geven", seed=63, contexts=ctx0, queries=[1] * len(ctx0),
                                pool_slack=120, page_size=64)
    b = workloads.generate(spec, dev, fill="zero")
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale, bound, 1,
                         out_dtype=torch.float32)
    tiles, _ = pa.select_tiles(pb)
    tiles.num_splits, tiles.variant = 4, 6
    workspace = torch.zeros(max(pa.workspace_size(pb, tiles), 256), dtype=torch.uint8,
                            device=dev)
    out = torch.empty(b.q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=dev)

    def step():
        pa.decode(b.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, spec.scale, bound,
                  out=out, lse=lse, tiles=tiles, workspace=workspace, problem=pb)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    # the pool holds 255 pages of 64 slots: every round's contexts fit in it
    _replay_rounds(b, g, out, lse, [ctx0, [1, 1, 4000, 3999, 0, 5], [2500] * 6], 300,
                   "graph even decode")


def test_short_runs_graph_replay(dev):
    """Speculative-decode verification (the short-run kernel, its even-work
    grid and per-unit merge) under capture; query lengths are fixed by the
    captured query_start_loc, contexts change between replays."""
    log("[graph short runs]")
    bound = 2500
    ql = [4, 4, 2, 4]
    ctx0 = [2500, 40, 900, 1300]
    spec = workloads.small_spec("gshort", seed=64, contexts=ctx0, queries=ql, pool_slack=150,
                                decode_layout=False)
    b = workloads.generate(spec, dev, fill="zero")
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale, bound,
                         max(ql), causal=True, out_dtype=torch.float32)
    tiles, ws = pa.select_tiles(pb)
    workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
    out = torch.empty(b.q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=dev)

    def step():
        pa.prefill(b.q, b.query_start_loc, b.k_pool, b.v_pool, b.block_tables, b.context_lens,
                   spec.scale, bound, max(ql), causal=True, out=out, lse=lse, tiles=tiles,
                   workspace=workspace, problem=pb)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    _replay_rounds(b, g, out, lse, [ctx0, [4, 2500, 2, 17], [2000, 2001, 2002, 4]], 400,
                   "graph short runs")


def test_noalloc_decode_graph_replay(dev):
    """pa_decode_noalloc captured in a graph, the use it exists for: no
    workspace argument, its partials in the library's per-GPU array (the
    first call, outside the capture, looks the array up)."""
    log("[graph noalloc decode]")
    bound = 3000
    ctx0 = [bound, 700, 1500]
    spec = workloads.small_spec("gnoalloc", seed=65, contexts=ctx0, queries=[1, 1, 1],
                                pool_slack=200)
    b = workloads.generate(spec, dev, fill="zero")
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, spec.scale, bound, 1,
                         out_dtype=torch.float32)
    tiles, _ = pa.select_tiles(pb)
    tiles.num_splits = 8
    out = torch.empty(b.q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=dev)

    def step():
        pa.decode_noalloc(b.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, spec.scale,
                          bound, out=out, lse=lse, tiles=tiles, problem=pb)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    _replay_rounds(b, g, out, lse, [ctx0, [17, 2999, 1], [0, 1024, 3000]], 500,
                   "graph noalloc decode")
