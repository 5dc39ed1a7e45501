"""A serving loop through the library: a prompt chunk, then decode steps.

Each step appends the step's new K/V rows into their pages
(pa_cache_append) and attends over the grown cache (pa_prefill for the
prompt chunk on its cached prefix, pa_decode for the single-token steps),
as a serving engine does with a paged prefix cache.  A host copy of the
pools follows every append through the oracle's own append, and every
step's output is compared with the oracle over that copy.  The contexts
cross page boundaries many times.  The second test captures one decode step
(append + attention) in a HIP graph and replays it with the lengths, the
queries and the new rows rewritten in place between replays.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_parity import bf16_allowance, dev, log  # noqa: F401

pytestmark = pytest.mark.gpu

PREFIX = [0, 40, 1000, 15, 300, 2047]   # cached tokens before the prompt chunk
CHUNK = [1, 90, 17, 33, 64, 1]          # prompt chunk tokens
STEPS = 40                              # decode steps after the chunk
HQ, HKV, D = 32, 8, 128


def _setup(dev, seed):
    prompt = [p + c for p, c in zip(PREFIX, CHUNK)]
    final = [L + STEPS for L in prompt]
    # pages for the whole horizon, as a serving allocator reserves them; the
    # slots past the current lengths hold stale values (NaN in the tails)
    spec = workloads.small_spec("serve", seed=seed, contexts=final, queries=[1] * len(final),
                                num_q_heads=HQ, num_kv_heads=HKV, head_dim=D)
    b = workloads.generate(spec, dev)
    host = [workloads.bf16_bits(b.k_pool), workloads.bf16_bits(b.v_pool)]
    return spec, b, prompt, final, host


def _randn_bf16(g, shape, dev):
    return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)


def _mirror_append(b, host, kn, vn, ctx, qsl):
    host[0], host[1] = oracle.append(host[0], host[1], b.spec.page_size, b.host_strides(),
                                     workloads.bf16_bits(kn), workloads.bf16_bits(vn),
                                     b.block_tables.cpu().numpy(), np.asarray(ctx, np.int32),
                                     None if qsl is None else np.asarray(qsl, np.int32))


def _check(b, host, q, ctx, qsl, out, label):
    inp = oracle.PagedInputs(q=workloads.bf16_bits(q), k_pool=host[0], v_pool=host[1],
                             block_tables=b.block_tables.cpu().numpy(),
                             context_lens=np.asarray(ctx, np.int32),
                             query_start_loc=None if qsl is None else np.asarray(qsl, np.int32),
                             num_kv_heads=HKV, page_size=b.spec.page_size,
                             strides=b.host_strides(), scale=b.spec.scale, causal=True)
    ref, _ = oracle.attention(inp)
    got = out.float().cpu().numpy().reshape(ref.shape)
    diff = np.abs(got - ref)
    if out.dtype == torch.float32:
        assert float(diff.max()) <= 2e-3, f"{label}: max|err| {diff.max()}"
    else:
        assert np.all(diff <= bf16_allowance(ref)), f"{label}: max|err| {diff.max()}"
    # the pools themselves: the library's appends equal the oracle's, bit for bit
    assert np.array_equal(workloads.bf16_bits(b.k_pool), host[0]), f"{label}: K pool"
    assert np.array_equal(workloads.bf16_bits(b.v_pool), host[1]), f"{label}: V pool"


def _prompt(dev, spec, b, prompt, host, g):
    qsl = [0] + list(np.cumsum(CHUNK))
    T = qsl[-1]
    q, kn, vn = (_randn_bf16(g, (T, HQ, D), dev), _randn_bf16(g, (T, HKV, D), dev),
                 _randn_bf16(g, (T, HKV, D), dev))
    ctx_d = torch.tensor(prompt, dtype=torch.int32, device=dev)
    qsl_d = torch.tensor(qsl, dtype=torch.int32, device=dev)
    pa.cache_append(kn, vn, b.k_pool, b.v_pool, b.block_tables, ctx_d, qsl_d)
    out = pa.prefill(q, qsl_d, b.k_pool, b.v_pool, b.block_tables, ctx_d, spec.scale,
                     max(prompt), max(CHUNK), out_dtype=torch.float32)
    torch.cuda.synchronize()
    _mirror_append(b, host, kn, vn, prompt, qsl)
    _check(b, host, q, prompt, qsl, out, "prompt chunk")


def test_serving_loop_eager(dev):
    """Prompt chunk, then 40 decode steps, each append + decode eagerly
    (bf16 output on odd steps, fp32 on even ones)."""
    log("[serving loop, eager]")
    spec, b, prompt, final, host = _setup(dev, 601)
    g = torch.Generator(device=dev)
    g.manual_seed(602)
    _prompt(dev, spec, b, prompt, host, g)
    B = len(prompt)
    ctx = list(prompt)
    for step in range(STEPS):
        ctx = [L + 1 for L in ctx]
        ctx_d = torch.tensor(ctx, dtype=torch.int32, device=dev)
        q = _randn_bf16(g, (B, HQ, D), dev)
        kn, vn = _randn_bf16(g, (B, HKV, D), dev), _randn_bf16(g, (B, HKV, D), dev)
        pa.cache_append(kn, vn, b.k_pool, b.v_pool, b.block_tables, ctx_d)
        dt = torch.float32 if step % 2 == 0 else torch.bfloat16
        out = pa.decode(q, b.k_pool, b.v_pool, b.block_tables, ctx_d, spec.scale, max(final),
                        out_dtype=dt)
        torch.cuda.synchronize()
        _mirror_append(b, host, kn, vn, ctx, None)
        _check(b, host, q, ctx, None, out, f"decode step {step}")


def test_serving_loop_graph(dev):
    """The decode step (append + decode, fixed launch shape and workspace)
    captured once and replayed 40 times with the lengths, the queries and
    the new rows rewritten in place between replays."""
    log("[serving loop, graph replay]")
    spec, b, prompt, final, host = _setup(dev, 611)
    g = torch.Generator(device=dev)
    g.manual_seed(612)
    _prompt(dev, spec, b, prompt, host, g)
    B = len(prompt)
    q_s = torch.zeros((B, HQ, D), dtype=torch.bfloat16, device=dev)
    k_s = torch.zeros((B, HKV, D), dtype=torch.bfloat16, device=dev)
    v_s = torch.zeros((B, HKV, D), dtype=torch.bfloat16, device=dev)
    ctx_d = torch.tensor(prompt, dtype=torch.int32, device=dev)
    out = torch.empty((B, HQ, D), dtype=torch.float32, device=dev)
    pb = pa.make_problem(q_s, b.k_pool, b.block_tables, B, spec.scale, max(final), 1,
                         out_dtype=torch.float32)
    tiles, ws_bytes = pa.select_tiles(pb)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def step():
        pa.cache_append(k_s, v_s, b.k_pool, b.v_pool, b.block_tables, ctx_d)
        pa.decode(q_s, b.k_pool, b.v_pool, b.block_tables, ctx_d, spec.scale, max(final),
                  out=out, tiles=tiles, workspace=ws, problem=pb)

    # a capture does not run its kernels: the pools are untouched until the
    # first replay
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    ctx = list(prompt)
    for i in range(STEPS):
        ctx = [L + 1 for L in ctx]
        ctx_d.copy_(torch.tensor(ctx, dtype=torch.int32))
        q_s.copy_(_randn_bf16(g, (B, HQ, D), dev))
        k_s.copy_(_randn_bf16(g, (B, HKV, D), dev))
        v_s.copy_(_randn_bf16(g, (B, HKV, D), dev))
        graph.replay()
        torch.cuda.synchronize()
        _mirror_append(b, host, k_s, v_s, ctx, None)
        _check(b, host, q_s, ctx, None, out, f"graph decode step {i}")
