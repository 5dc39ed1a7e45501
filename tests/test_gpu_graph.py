"""HIP-graph capture and replay (the static launch grid + graphs steps of the
IBM Triton summary's five-step list): a decode step and a mixed prefill step
are captured once; lengths, block tables and queries are then rewritten in
place (within the capture-time bounds) and every replay is checked against
the oracle.  Eager work and synchronisations run between replays, and a
repeated replay must reproduce the same bits."""
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
