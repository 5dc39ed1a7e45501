"""pa_decode_noalloc, the variant of pa_decode for callers that cannot
allocate (its partials live in the library's per-GPU scratch array), against
pa_decode with a caller workspace: the same kernels and launch shape, so the
outputs must be identical bit for bit, and both within the oracle bar.
Calls follow each other on one GPU with shrinking inputs and changing launch
shapes, so each call runs over whatever the previous one left in the array.
"""
import ctypes

import numpy as np
import pytest
import torch

from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_parity import compare, dev, log  # noqa: F401

pytestmark = pytest.mark.gpu


def _tiles(b, splits=None, variant=None, waves=None):
    pb = pa.make_problem(b.q, b.k_pool, b.block_tables, b.num_seqs, b.spec.scale,
                         b.max_context_len, 1, out_dtype=torch.float32)
    t, _ = pa.select_tiles(pb)
    if splits is not None:
        t.num_splits = splits
    if variant is not None:
        t.variant = variant
    if waves is not None:
        t.waves_per_wg = waves
    return pb, t


def _both(b, label, rows=None, **kw):
    """pa_decode (fresh zeroed workspace) and pa_decode_noalloc on one batch:
    identical bits, and the result within the oracle bar."""
    pb, t = _tiles(b, **kw)
    ws_bytes = pa.workspace_size(pb, t)
    assert ws_bytes <= pa.NOALLOC_SCRATCH_BYTES
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=b.q.device)
    shape = b.q.shape
    out1 = torch.empty(shape, dtype=torch.float32, device=b.q.device)
    lse1 = torch.empty(shape[:2], dtype=torch.float32, device=b.q.device)
    out2 = torch.full(shape, float("nan"), dtype=torch.float32, device=b.q.device)
    lse2 = torch.full(shape[:2], float("nan"), dtype=torch.float32, device=b.q.device)
    pa.decode(b.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, b.spec.scale,
              b.max_context_len, out=out1, lse=lse1, tiles=t, workspace=ws, problem=pb)
    pa.decode_noalloc(b.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, b.spec.scale,
                      b.max_context_len, out=out2, lse=lse2, tiles=t, problem=pb)
    torch.cuda.synchronize()
    log(f"{label}: tiles {t.as_dict()}, workspace {ws_bytes} B")
    assert torch.equal(out1, out2), f"{label}: outputs differ from pa_decode's"
    assert torch.equal(lse1, lse2), f"{label}: LSEs differ from pa_decode's"
    compare(b, out2, lse2, rows=rows, label=label)


def _varied(name, seed, n, lo, hi):
    rng = np.random.default_rng(seed)
    ctx = [int(x) for x in rng.integers(lo, hi + 1, size=n)]
    return workloads.small_spec(name, seed=seed, contexts=ctx, queries=[1] * n, pool_slack=50)


def test_noalloc_two_calls_shrinking(dev):
    """A 64-sequence batch on the table's launch shape (even-work grid), then
    a 3-sequence batch with more splits: each equals pa_decode."""
    log("[noalloc: 64 sequences, then 3]")
    big = workloads.generate(_varied("noalloc_big", 11, 64, 128, 8192), dev)
    rng = np.random.default_rng(5)
    n = big.num_seqs * big.spec.num_q_heads
    rows = np.union1d(rng.choice(n, 256, replace=False), [0, n - 1])
    _both(big, "noalloc big (table)", rows=rows)
    small = workloads.generate(
        workloads.small_spec("noalloc_small", seed=12, contexts=[3000, 0, 517],
                             queries=[1, 1, 1]), dev)
    _both(small, "noalloc small (S=48, even)", splits=48, variant=6)


def test_noalloc_fused_merge_after_other_calls(dev):
    """The fused last-workgroup merge (variant 0) needs zeroed arrival
    counters; the previous calls left partial outputs where they now sit."""
    log("[noalloc: fused merge after other calls]")
    a = workloads.generate(_varied("noalloc_a", 21, 16, 1000, 6000), dev)
    _both(a, "noalloc a (S=64, even)", splits=64, variant=6)
    b = workloads.generate(
        workloads.small_spec("noalloc_b", seed=22, contexts=[5000, 40, 2049, 1],
                             queries=[1, 1, 1, 1]), dev)
    for S in (7, 32):
        _both(b, f"noalloc b (S={S}, fused)", splits=S, variant=0, waves=8)
        _both(b, f"noalloc b (S={S}, separate)", splits=S, variant=2, waves=4)


def test_noalloc_short_run_kernel(dev):
    """Decode at G = 32 (32 query heads on one KV head) runs on the short-run
    kernel, whose (token, head) partials also live in the array."""
    log("[noalloc: G = 32]")
    b = workloads.generate(
        workloads.small_spec("noalloc_g32", seed=31, contexts=[9000, 300, 1], queries=[1, 1, 1],
                             num_q_heads=32, num_kv_heads=1), dev)
    _both(b, "noalloc G=32 (table)")
    _both(b, "noalloc G=32 (S=5)", splits=5)


def test_noalloc_rejects_oversize(dev):
    """A launch shape whose workspace exceeds the array is refused before
    anything is enqueued (256 sequences at 8k context, 128 splits)."""
    lib = pa.load()
    pb = pa.Problem()
    for k, v in dict(num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                     max_blocks_per_seq=512, kv_stride_page=16 * 8 * 128,
                     kv_stride_token=8 * 128, kv_stride_head=128, max_context_len=8192,
                     max_query_len=1, total_query_tokens=256, causal=1,
                     scale=0.08838834764831845, out_dtype=pa.PA_BF16).items():
        setattr(pb, k, v)
    t, _ = pa.select_tiles(pb)
    t.num_splits, t.variant = 128, 6
    need = pa.workspace_size(pb, t)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(4096, dtype=torch.uint8, device=dev)  # never read: the check comes first
    p = ctypes.c_void_p(buf.data_ptr())
    st = lib.pa_decode_noalloc(ctypes.byref(pb), ctypes.byref(t), p, p, p, p, p, p, None,
                               ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == pa.PA_ERR_WORKSPACE
    torch.cuda.synchronize()
