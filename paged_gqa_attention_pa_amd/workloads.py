"""Seeded synthetic inputs for paged GQA attention.

This module only draws and lays out inputs; it holds none of the attention
arithmetic, so both the HIP path and the fp64 oracle can consume what it
produces.  Shapes follow Llama-3.1-8B attention (32 query heads, 8 KV heads,
head_dim 128), the model the IBM Triton paged-attention summary reports on
("一行 Triton 代码同时跑赢 NVIDIA 和 AMD…", section on where it already runs);
no model weights are involved.

Recipe (every draw from one seeded torch.Generator, in this order):
  1. lengths (context lengths and query lengths),
  2. block tables: disjoint slices of one randperm of the page pool, padded
     with -1,
  3. Q, then K, then V: fp32 standard normal, rounded to bf16 (RNE),
     K and V drawn only for the pages a block table references.
Pages no table references, and the slots past each context in its last page,
are filled with NaN (parity tests) or zero (benchmark): no result may depend
on them.

The default paged layout is [num_pages, page_size, num_kv_heads, head_dim]
(token-major inside a page); Q and the output are packed [tokens, Hq, D].
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    """One synthetic workload.

    context_lens / query_lens are either explicit lists or drawn: when
    ``ctx_range`` is set, ``num_draw`` context lengths are drawn uniformly in
    [lo, hi] (inclusive) and come first in the batch, with query length
    ``draw_query_len`` (1: decode; a few tokens: speculative-decode
    verification); ``fixed`` lists (context_len, query_len) pairs appended
    after them.
    """
    name: str
    seed: int
    pool_pages: int
    fixed: Sequence[tuple] = ()
    ctx_range: Optional[tuple] = None
    num_draw: int = 0
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    page_size: int = 16
    causal: bool = True
    max_blocks: Optional[int] = None   # block-table row stride; default = bound
    decode_layout: bool = False        # every query length 1 -> no query_start_loc
    logit_gain: float = 1.0            # multiplies Q after drawing (stress cases)
    draw_query_len: int = 1            # query tokens of each drawn sequence

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


# The workloads: Llama-3.1-8B-shaped attention, bf16, page size 16.
WORKLOADS = {
    # single decode step, batch 1, context 512
    "decode_ctx512": WorkloadSpec(
        name="decode_ctx512", seed=1001, pool_pages=64, fixed=[(512, 1)],
        decode_layout=True),
    # long-context decode, batch 1, context 32768 in a 4096-page pool
    "decode_ctx32k": WorkloadSpec(
        name="decode_ctx32k", seed=1002, pool_pages=4096, fixed=[(32768, 1)],
        decode_layout=True),
    # batched decode, 64 sequences, contexts uniform in [128, 8192]
    "decode_b64": WorkloadSpec(
        name="decode_b64", seed=1003, pool_pages=40000, ctx_range=(128, 8192),
        num_draw=64, max_blocks=512, decode_layout=True),
    # causal chunked prefill: 4 x (1024 cached + 2048 new tokens)
    "prefill_chunk2048": WorkloadSpec(
        name="prefill_chunk2048", seed=1004, pool_pages=1024,
        fixed=[(3072, 2048)] * 4),
    # mixed batch: 16 decodes, contexts in [512, 16384], then 2 prefill
    # chunks of 512 new tokens on 4096-token prefixes, one launch
    "mixed_unified": WorkloadSpec(
        name="mixed_unified", seed=1005, pool_pages=40000, ctx_range=(512, 16384),
        num_draw=16, fixed=[(4608, 512)] * 2, max_blocks=1024),
    # speculative-decode verification: 64 sequences, contexts U[128, 8192],
    # 4 causal query tokens each (3 drafted + 1), one pa_prefill launch
    "spec_verify_b64": WorkloadSpec(
        name="spec_verify_b64", seed=1006, pool_pages=40000, ctx_range=(128, 8192),
        num_draw=64, max_blocks=512, draw_query_len=4),
    # large decode batch: 256 sequences of 8192 tokens (8 GiB of K/V), the
    # steady-state streaming rate with no per-step start-up to amortise
    "decode_b256_ctx8k": WorkloadSpec(
        name="decode_b256_ctx8k", seed=1007, pool_pages=256 * 512 + 64,
        fixed=[(8192, 1)] * 256, decode_layout=True),
}
WORKLOAD_ORDER = ["decode_ctx512", "decode_ctx32k", "decode_b64",
                  "prefill_chunk2048", "mixed_unified", "spec_verify_b64"]


@dataclasses.dataclass
class Batch:
    spec: WorkloadSpec
    q: torch.Tensor                 # [T, Hq, D] bf16
    k_pool: torch.Tensor            # [pool_pages, P, Hkv, D] bf16
    v_pool: torch.Tensor
    block_tables: torch.Tensor      # [B, max_blocks] int32, -1 padded
    context_lens: torch.Tensor      # [B] int32
    query_start_loc: Optional[torch.Tensor]  # [B+1] int32; None for decode layout
    query_lens: List[int]
    used_pages: torch.Tensor        # [n_used] int64 page ids in table order

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.numel())

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max().item()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return max(self.query_lens) if self.query_lens else 0

    def kv_strides(self):
        """(page, token, head) strides in elements of both pools."""
        s = self.k_pool.stride()
        return int(s[0]), int(s[1]), int(s[2])

    def host_strides(self):
        """(page, token, head) strides of the pools' host copies (bf16_bits
        copies them in logical [page, slot, head, dim] order, contiguous),
        whatever order the device pools store their pages in."""
        _, P, Hkv, D = self.k_pool.shape
        return P * Hkv * D, Hkv * D, D


def _lengths(spec: WorkloadSpec, g: torch.Generator):
    ctx, ql = [], []
    if spec.ctx_range is not None and spec.num_draw > 0:
        lo, hi = spec.ctx_range
        drawn = torch.randint(lo, hi + 1, (spec.num_draw,), generator=g, device=g.device)
        ctx += [int(x) for x in drawn.cpu()]
        ql += [spec.draw_query_len] * spec.num_draw
    for c, q in spec.fixed:
        ctx.append(int(c))
        ql.append(int(q))
    return ctx, ql


def plan(spec: WorkloadSpec, device="cpu", g: Optional[torch.Generator] = None):
    """Draw steps 1-2 (lengths, block tables) of ``spec``.

    Returns (context_lens, query_lens, block_tables [B, max_blocks] int32,
    used page ids in table order, pages needed per sequence, generator).
    """
    device = torch.device(device)
    if g is None:
        g = torch.Generator(device=device)
        g.manual_seed(spec.seed)
    P = spec.page_size
    if spec.num_q_heads % spec.num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    ctx, ql = _lengths(spec, g)
    B = len(ctx)
    for c, q in zip(ctx, ql):
        if c < 0 or q < 0:
            raise ValueError(f"bad (context, query) length pair ({c}, {q})")
    pages_needed = [-(-c // P) for c in ctx]
    bound = max(pages_needed) if pages_needed else 0
    max_blocks = spec.max_blocks if spec.max_blocks is not None else max(bound, 1)
    if bound > max_blocks:
        raise ValueError("a context needs more pages than max_blocks")
    n_used = sum(pages_needed)
    if n_used > spec.pool_pages:
        raise ValueError("page pool too small for the drawn contexts")
    perm = torch.randperm(spec.pool_pages, generator=g, device=device)
    bt = torch.full((B, max_blocks), -1, dtype=torch.int32, device=device)
    off = 0
    for s, n in enumerate(pages_needed):
        bt[s, :n] = perm[off:off + n].to(torch.int32)
        off += n
    used = perm[:n_used].to(torch.int64)
    return ctx, ql, bt, used, pages_needed, g


def generate(spec: WorkloadSpec, device="cpu", fill: str = "nan") -> Batch:
    """Draw one batch of ``spec`` on ``device`` (generator on that device).

    fill: "nan" poisons every page slot no context covers, "zero" zeroes them.
    The same (spec, device type) always yields the same bits.
    """
    if fill not in ("nan", "zero"):
        raise ValueError("fill must be 'nan' or 'zero'")
    device = torch.device(device)
    P, Hq, Hkv, D = spec.page_size, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    # 1-2. lengths, block tables
    ctx, ql, bt, used, pages_needed, g = plan(spec, device)
    n_used = int(used.numel())

    # 3. Q, K, V
    T = sum(ql)
    q = torch.randn((T, Hq, D), generator=g, device=device, dtype=torch.float32)
    if spec.logit_gain != 1.0:
        q = q * spec.logit_gain
    q = q.to(torch.bfloat16)
    fill_val = float("nan") if fill == "nan" else 0.0
    pools = []
    for _ in range(2):
        vals = torch.randn((n_used, P, Hkv, D), generator=g, device=device,
                           dtype=torch.float32).to(torch.bfloat16)
        pool = torch.full((spec.pool_pages, P, Hkv, D), fill_val, dtype=torch.bfloat16,
                          device=device)
        if n_used:
            pool[used] = vals
        pools.append(pool)
    k_pool, v_pool = pools

    # slots past each context in its last page hold stale data too
    off = 0
    for s, n in enumerate(pages_needed):
        tail = ctx[s] - (n - 1) * P
        if n and tail < P:
            last = used[off + n - 1]
            k_pool[last, tail:] = fill_val
            v_pool[last, tail:] = fill_val
        off += n

    qsl = None
    if not spec.decode_layout:
        qsl = torch.tensor([0] + list(np.cumsum(ql)), dtype=torch.int32, device=device)
    elif any(x != 1 for x in ql):
        raise ValueError("decode layout needs query length 1 everywhere")
    return Batch(spec=spec, q=q, k_pool=k_pool, v_pool=v_pool, block_tables=bt,
                 context_lens=torch.tensor(ctx, dtype=torch.int32, device=device),
                 query_start_loc=qsl, query_lens=ql, used_pages=used)


# How the pools store a page: token_major keeps the generated order
# [page][slot][kv head][dim] (one token's heads side by side); head_major
# stores [page][kv head][slot][dim] (one head's slots side by side, so a 16-key
# tile of a head is one contiguous 4 KiB run at D = 128).  Both are seen
# through the same logical [page, slot, head, dim] tensor, with other strides.
KV_LAYOUTS = ("token_major", "head_major")


def with_layout(batch: Batch, layout: str) -> Batch:
    """The batch with its pools stored in `layout` (same values)."""
    if layout == "token_major":
        return batch
    if layout != "head_major":
        raise ValueError(f"layout must be one of {KV_LAYOUTS}")

    def head_major(t):
        return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)

    return dataclasses.replace(batch, k_pool=head_major(batch.k_pool),
                               v_pool=head_major(batch.v_pool))


def new_kv(batch: Batch, seed: int):
    """K and V rows of a batch's new tokens, as a paged append takes them:
    bf16 [T, Hkv, D] each, fp32 standard normal rounded to bf16, K first,
    from a generator seeded with ``seed`` on the batch's device."""
    dev = batch.q.device
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    shape = (batch.num_tokens, batch.spec.num_kv_heads, batch.spec.head_dim)
    k = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return k, v


def small_spec(name: str, seed: int, contexts: Sequence[int], queries: Sequence[int],
               num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
               causal=True, pool_slack=7, decode_layout=None, logit_gain=1.0,
               max_blocks=None) -> WorkloadSpec:
    """A fixed-length workload for tests (pool = used pages + slack)."""
    pages = sum(-(-c // page_size) for c in contexts)
    if decode_layout is None:
        decode_layout = all(q == 1 for q in queries)
    return WorkloadSpec(name=name, seed=seed, pool_pages=pages + pool_slack,
                        fixed=list(zip(contexts, queries)), num_q_heads=num_q_heads,
                        num_kv_heads=num_kv_heads, head_dim=head_dim,
                        page_size=page_size, causal=causal,
                        decode_layout=decode_layout, logit_gain=logit_gain,
                        max_blocks=max_blocks)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a bf16 tensor's bits (copies to host if needed)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
