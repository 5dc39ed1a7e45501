"""The seeded input generator (CPU)."""
import math

import numpy as np
import pytest
import torch

from paged_gqa_attention_pa_amd import workloads


def _small():
    return workloads.small_spec("t", seed=5, contexts=[1, 16, 17, 100, 0], queries=[1, 1, 5, 30, 0],
                                num_q_heads=8, num_kv_heads=2, head_dim=32, pool_slack=9)


def test_same_seed_same_bits():
    a = workloads.generate(_small(), "cpu")
    b = workloads.generate(_small(), "cpu")
    for x, y in [(a.q, b.q), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool)]:
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(a.block_tables, b.block_tables)
    assert torch.equal(a.query_start_loc, b.query_start_loc)


def test_tables_disjoint_in_range_and_poisoned():
    spec = _small()
    b = workloads.generate(spec, "cpu", fill="nan")
    bt = b.block_tables.numpy()
    P = spec.page_size
    ids = []
    for s, L in enumerate(b.context_lens.tolist()):
        n = -(-L // P)
        assert np.all(bt[s, n:] == -1)
        ids += bt[s, :n].tolist()
        for j in range(n):  # covered slots are finite, the tail of the last page is NaN
            page = bt[s, j]
            filled = min(P, L - j * P)
            assert torch.isfinite(b.k_pool[page, :filled].float()).all()
            assert torch.isnan(b.v_pool[page, filled:].float()).all()
    assert len(ids) == len(set(ids))
    assert all(0 <= i < spec.pool_pages for i in ids)
    unused = sorted(set(range(spec.pool_pages)) - set(ids))
    assert torch.isnan(b.k_pool[unused].float()).all()
    qsl = b.query_start_loc.numpy()
    assert qsl[0] == 0 and np.all(np.diff(qsl) == np.array(b.query_lens))
    assert qsl[-1] == b.q.shape[0]


def test_zero_fill():
    b = workloads.generate(_small(), "cpu", fill="zero")
    assert torch.isfinite(b.k_pool.float()).all() and torch.isfinite(b.v_pool.float()).all()


def test_values_are_standard_normal_bf16():
    spec = workloads.small_spec("n", seed=6, contexts=[4096], queries=[1], pool_slack=0)
    b = workloads.generate(spec, "cpu")
    k = b.k_pool.float()
    assert abs(k.mean().item()) < 0.01 and abs(k.std().item() - 1) < 0.01
    # bf16 round trip is exact
    assert torch.equal(b.q.float().to(torch.bfloat16).view(torch.int16), b.q.view(torch.int16))


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER)
def test_named_workload_plans(name):
    spec = workloads.WORKLOADS[name]
    ctx, ql, bt, used, pages, _ = workloads.plan(spec, "cpu")
    assert spec.num_q_heads == 32 and spec.num_kv_heads == 8 and spec.head_dim == 128
    assert spec.page_size == 16
    assert spec.scale == np.float32(1 / math.sqrt(128))
    assert len(set(used.tolist())) == used.numel() <= spec.pool_pages
    if name == "decode_ctx512":
        assert ctx == [512] and ql == [1] and spec.pool_pages == 64
    if name == "decode_ctx32k":
        assert ctx == [32768] and spec.pool_pages == 4096
    if name == "decode_b64":
        assert len(ctx) == 64 and min(ctx) >= 128 and max(ctx) <= 8192 and set(ql) == {1}
        assert bt.shape == (64, 512)
    if name == "prefill_chunk2048":
        assert ctx == [3072] * 4 and ql == [2048] * 4
    if name == "mixed_unified":
        assert len(ctx) == 18 and ql[:16] == [1] * 16 and ql[16:] == [512, 512]
        assert min(ctx[:16]) >= 512 and max(ctx[:16]) <= 16384 and ctx[16:] == [4608, 4608]


def test_head_major_layout_keeps_values():
    """with_layout stores each page head by head without changing a value:
    the logical pools are equal, the strides are head-major, and the oracle
    gives the same bits from the storage of either layout read with its own
    strides."""
    import oracle
    spec = workloads.small_spec("hm", seed=21, contexts=[40, 17, 1], queries=[5, 17, 1],
                                num_q_heads=8, num_kv_heads=2, head_dim=64,
                                decode_layout=False)
    b = workloads.generate(spec, "cpu")
    h = workloads.with_layout(b, "head_major")
    assert workloads.with_layout(b, "token_major") is b
    assert torch.equal(h.k_pool.view(torch.int16), b.k_pool.view(torch.int16))
    assert torch.equal(h.v_pool.view(torch.int16), b.v_pool.view(torch.int16))
    npg, P, Hkv, D = b.k_pool.shape
    assert h.kv_strides() == (P * Hkv * D, D, P * D)
    assert h.host_strides() == b.host_strides() == (P * Hkv * D, Hkv * D, D)
    outs = []
    for bb in (b, h):
        # the storage itself, as the device kernels read it
        store = lambda t: t.permute(0, 2, 1, 3).contiguous() if bb is h else t  # noqa: E731
        inp = oracle.PagedInputs(
            q=workloads.bf16_bits(bb.q), k_pool=workloads.bf16_bits(store(bb.k_pool)),
            v_pool=workloads.bf16_bits(store(bb.v_pool)),
            block_tables=bb.block_tables.numpy(), context_lens=bb.context_lens.numpy(),
            query_start_loc=bb.query_start_loc.numpy(), num_kv_heads=Hkv, page_size=P,
            strides=bb.kv_strides(), scale=spec.scale, causal=True)
        outs.append(oracle.attention(inp))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    with pytest.raises(ValueError):
        workloads.with_layout(b, "slot_major")
