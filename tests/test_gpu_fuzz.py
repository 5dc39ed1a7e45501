"""Seeded random problems through pa_decode and pa_prefill against the fp64
oracle: random query-head groups (G = 1..32), head dims (64, 128, 256),
batch sizes, length mixes (empty sequences, single tokens, short runs,
chunks on cached prefixes, a few past 32k keys), causal or not, bf16 or fp32 outputs, with or
without the LSE, pools in the default layout or seen through other strides
(head-major storage, or padded rows and heads holding NaN), pages of 16 to
256 slots, and sometimes a forced split count over a NaN-filled workspace.  Each case goes through
whatever kernels the host picks for it (decode kernels, short-run kernel,
query tiles with or without decode workgroups, tile splits), so the routing
is exercised on shapes no hand-written case names.  Long rows are compared
on a seeded sample of output rows.  The paged append gets the same random
batches and pool layouts, compared bit for bit.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_parity import compare, dev, log, run_decode, run_prefill  # noqa: F401

pytestmark = pytest.mark.gpu

# PA_FUZZ_CASES raises the count for a wider one-off sweep
N_CASES = int(os.environ.get("PA_FUZZ_CASES", "200"))
MAX_ROWS = 384  # output rows checked per case (sampled beyond this)


def draw_case(i):
    rng = np.random.default_rng(7100 + i)
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    while G * hkv > 64:
        hkv //= 2
    D = int(rng.choice([64, 128, 128, 256]))
    B = int(rng.integers(1, 6))
    mode = rng.choice(["decode", "short", "mixed", "chunks"])
    ctx, ql = [], []
    for _ in range(B):
        kind = mode if mode != "mixed" else rng.choice(["decode", "short", "chunk", "empty"])
        if kind == "decode":
            q = 1
        elif kind == "short":
            q = int(rng.integers(2, 17))
        elif kind == "empty":
            q = 0
        else:
            q = int(rng.integers(17, 200))
        # rarely past 32k keys, where the LDS window of block offsets is restaged
        prefix = 0 if q == 0 else int(rng.choice([0, rng.integers(0, 600), rng.integers(0, 3000),
                                                  rng.integers(0, 3000),
                                                  rng.integers(0, 3000) + 33000 * (i % 7 == 0)]))
        ctx.append(q + prefix)
        ql.append(q)
    if all(q == 0 for q in ql):
        ctx[0], ql[0] = 40, 1
    if D == 256 and i % 4 != 0:
        # mostly short-run shapes at 256 (runs of up to 32 rows, the
        # short-run kernel); every fourth case keeps its longer runs (the
        # query tiles)
        cap = max(1, 32 // G)
        for k in range(B):
            if ql[k] > cap:
                ctx[k] -= ql[k] - cap
                ql[k] = cap
    causal = bool(rng.integers(0, 4) > 0)
    out_dtype = torch.float32 if rng.integers(0, 3) == 0 else torch.bfloat16
    decode_layout = all(q == 1 for q in ql) and bool(rng.integers(0, 2))
    layout = str(rng.choice(["default", "default", "head_major", "padded"]))
    with_lse = bool(rng.integers(0, 3) > 0)
    force = int(rng.choice([0, 0, 0, 2, 3, 8]))  # splits (decode) / tile splits (prefill)
    # drawn last, so the fields above are those of the 16-slot-page cases
    P = int(rng.choice([16, 16, 16, 32, 64, 256]))
    return dict(G=G, hkv=hkv, D=D, ctx=ctx, ql=ql, causal=causal, out_dtype=out_dtype,
                decode_layout=decode_layout, layout=layout, with_lse=with_lse, force=force,
                P=P, seed=7100 + i)


def strided_pools(b, layout):
    """The batch's pools seen through other strides, same logical contents."""
    if layout == "head_major":
        ks = b.k_pool.permute(0, 2, 1, 3).contiguous()
        vs = b.v_pool.permute(0, 2, 1, 3).contiguous()
        return ks.permute(0, 2, 1, 3), vs.permute(0, 2, 1, 3)
    npg, P, Hkv, D = b.k_pool.shape
    ks = torch.full((npg, P, Hkv + 1, D + 8), float("nan"), dtype=b.k_pool.dtype,
                    device=b.k_pool.device)
    vs = ks.clone()
    ks[:, :, :Hkv, :D] = b.k_pool
    vs[:, :, :Hkv, :D] = b.v_pool
    return ks[:, :, :Hkv, :D], vs[:, :, :Hkv, :D]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_problem(dev, i):
    c = draw_case(i)
    log(f"[fuzz {i}] G={c['G']} Hkv={c['hkv']} D={c['D']} ctx={c['ctx']} q={c['ql']} "
        f"causal={c['causal']} {c['out_dtype']} decode_layout={c['decode_layout']} "
        f"layout={c['layout']} lse={c['with_lse']} force={c['force']} P={c['P']}")
    spec = workloads.small_spec(f"fuzz{i}", c["seed"], c["ctx"], c["ql"],
                                num_q_heads=c["G"] * c["hkv"], num_kv_heads=c["hkv"],
                                head_dim=c["D"], causal=c["causal"],
                                decode_layout=c["decode_layout"], page_size=c["P"])
    b = workloads.generate(spec, dev)
    bg = b  # what the GPU sees; the oracle reads b's default layout
    if c["layout"] != "default":
        kv, vv = strided_pools(b, c["layout"])
        bg = dataclasses.replace(b, k_pool=kv, v_pool=vv)
    force = c["force"] or None
    if c["decode_layout"]:
        out, lse = run_decode(bg, c["out_dtype"], splits=force, with_lse=c["with_lse"])
    else:
        out, lse = run_prefill(bg, c["out_dtype"], with_lse=c["with_lse"],
                               tile_splits=force if max(c["ql"]) > 1 else None,
                               stale_workspace=force is not None)
    T = out.shape[0] * out.shape[1]
    rows = None
    if T > MAX_ROWS:
        rows = np.sort(np.random.default_rng(c["seed"]).choice(T, MAX_ROWS, replace=False))
    compare(b, out, lse, rows=rows, label=f"fuzz {i}")


N_APPEND = 60


def storage_pools(b, layout):
    """(storage K, storage V, view K, view V, strides) for a pool layout:
    the views are what the library is handed, the storage is what the
    oracle reads through the same strides."""
    if layout == "default":
        return b.k_pool, b.v_pool, b.k_pool, b.v_pool, b.kv_strides()
    npg, P, Hkv, D = b.k_pool.shape
    if layout == "head_major":
        ks = b.k_pool.permute(0, 2, 1, 3).contiguous()
        vs = b.v_pool.permute(0, 2, 1, 3).contiguous()
        kv, vv = ks.permute(0, 2, 1, 3), vs.permute(0, 2, 1, 3)
    else:
        ks = torch.full((npg, P, Hkv + 1, D + 8), float("nan"), dtype=b.k_pool.dtype,
                        device=b.k_pool.device)
        vs = ks.clone()
        ks[:, :, :Hkv, :D] = b.k_pool
        vs[:, :, :Hkv, :D] = b.v_pool
        kv, vv = ks[:, :, :Hkv, :D], vs[:, :, :Hkv, :D]
    return ks, vs, kv, vv, tuple(int(x) for x in kv.stride()[:3])


@pytest.mark.parametrize("i", range(N_APPEND))
def test_random_append(dev, i):
    """pa_cache_append on random batches and pool layouts, bit for bit
    against the oracle's append over the whole pool."""
    c = draw_case(1000 + i)
    log(f"[fuzz append {i}] Hkv={c['hkv']} D={c['D']} ctx={c['ctx']} q={c['ql']} "
        f"decode_layout={c['decode_layout']} layout={c['layout']}")
    spec = workloads.small_spec(f"fuzz_app{i}", c["seed"], c["ctx"], c["ql"],
                                num_q_heads=c["G"] * c["hkv"], num_kv_heads=c["hkv"],
                                head_dim=c["D"], causal=c["causal"],
                                decode_layout=c["decode_layout"])
    b = workloads.generate(spec, dev)
    kn, vn = workloads.new_kv(b, seed=c["seed"] + 1)
    ks, vs, kv, vv, strides = storage_pools(b, c["layout"])
    qsl = b.query_start_loc
    k_exp, v_exp = oracle.append(
        workloads.bf16_bits(ks), workloads.bf16_bits(vs), spec.page_size, strides,
        workloads.bf16_bits(kn), workloads.bf16_bits(vn), b.block_tables.cpu().numpy(),
        b.context_lens.cpu().numpy(), None if qsl is None else qsl.cpu().numpy())
    pa.cache_append(kn, vn, kv, vv, b.block_tables, b.context_lens, qsl)
    torch.cuda.synchronize()
    assert np.array_equal(workloads.bf16_bits(ks), k_exp), "K pool differs from the oracle"
    assert np.array_equal(workloads.bf16_bits(vs), v_exp), "V pool differs from the oracle"
