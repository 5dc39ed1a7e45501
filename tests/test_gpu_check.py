"""pa_check_inputs on the GPU: consistent batches report nothing; each kind
of bad table or length, planted in a copy of a valid batch, reports its own
bit and no other.  The check kernel only reads the tables, so the planted
values are safe to run."""
import pytest
import torch

from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_parity import dev, log  # noqa: F401

pytestmark = pytest.mark.gpu


def _batch(dev, decode_layout):
    if decode_layout:
        spec = workloads.small_spec("chk_dec", 61, [700, 33, 1, 5, 2049], [1, 1, 1, 1, 1])
    else:
        spec = workloads.small_spec("chk_pre", 62, [300, 77, 1000, 0, 40], [140, 77, 1, 0, 40])
    return workloads.generate(spec, dev)


def _flags(b, bt=None, ctx=None, qsl="same", max_ctx=None, max_q=None, num_pages=None):
    bt = b.block_tables if bt is None else bt
    ctx = b.context_lens if ctx is None else ctx
    qsl = b.query_start_loc if qsl == "same" else qsl
    pb = pa.make_problem(b.q, b.k_pool, bt, b.num_seqs, b.spec.scale,
                         b.max_context_len if max_ctx is None else max_ctx,
                         (b.max_query_len if qsl is not None else 1) if max_q is None else max_q)
    pages = b.k_pool.shape[0] if num_pages is None else num_pages
    return pa.check_inputs(pb, pages, bt, ctx, qsl)


@pytest.mark.parametrize("decode_layout", [True, False], ids=["decode", "prefill"])
def test_check_consistent(dev, decode_layout):
    log(f"[check consistent decode_layout={decode_layout}]")
    b = _batch(dev, decode_layout)
    assert _flags(b) == 0


def test_check_empty_context_decode(dev):
    """A decode row of an empty context has a query token and no position
    for it: defined for attention (the row sees no key), undefined for an
    append, and reported as such."""
    log("[check empty context]")
    b = _batch(dev, True)
    ctx = b.context_lens.clone()
    ctx[3] = 0
    assert _flags(b, ctx=ctx) == pa.CHECK_CONTEXT_SHORT


@pytest.mark.parametrize("decode_layout", [True, False], ids=["decode", "prefill"])
def test_check_bad_pages(dev, decode_layout):
    log(f"[check bad pages decode_layout={decode_layout}]")
    b = _batch(dev, decode_layout)
    npg = b.k_pool.shape[0]
    for bad in (npg, -1, 1 << 30):
        bt = b.block_tables.clone()
        bt[0, 1] = bad  # sequence 0 uses more than one page
        assert _flags(b, bt=bt) == pa.CHECK_PAGE
    # entries past a context's last page are never read: anything goes there
    bt = b.block_tables.clone()
    L0 = int(b.context_lens[0])
    bt[0, (L0 + 15) // 16:] = npg + 5
    assert _flags(b, bt=bt) == 0
    # a pool said to be smaller than the pages in use
    used_max = int(b.block_tables.max())
    assert _flags(b, num_pages=used_max) == pa.CHECK_PAGE


def test_check_context_bounds(dev):
    log("[check context bounds]")
    b = _batch(dev, True)
    # a host bound below the longest context
    assert _flags(b, max_ctx=b.max_context_len - 1) == pa.CHECK_CONTEXT_BOUND
    # a negative length
    ctx = b.context_lens.clone()
    ctx[2] = -3
    assert _flags(b, ctx=ctx) == pa.CHECK_CONTEXT_BOUND | pa.CHECK_CONTEXT_SHORT
    # a context longer than its table row (the host bound is at most a full
    # row, so this is past the bound as well)
    ctx, bt = b.context_lens.clone(), b.block_tables.clone()
    rows = b.block_tables.shape[1]
    ctx[1] = rows * 16 + 1
    assert _flags(b, ctx=ctx) == (pa.CHECK_CONTEXT_BLOCKS | pa.CHECK_CONTEXT_BOUND |
                                  pa.CHECK_PAGE)  # its padded entries are now in use
    bt[1, :] = 0  # a full row of valid pages
    assert _flags(b, bt=bt, ctx=ctx) == pa.CHECK_CONTEXT_BLOCKS | pa.CHECK_CONTEXT_BOUND


def test_check_query_starts(dev):
    log("[check query starts]")
    b = _batch(dev, False)
    qsl = b.query_start_loc.clone()
    qsl[2] = qsl[1] - 1  # falls
    f = _flags(b, qsl=qsl)
    assert f & pa.CHECK_QUERY_STARTS and not f & pa.CHECK_PAGE
    qsl = b.query_start_loc.clone()
    qsl[0] = 1  # does not start at 0
    assert _flags(b, qsl=qsl) & pa.CHECK_QUERY_STARTS
    qsl = b.query_start_loc.clone()
    qsl[-1] -= 1  # does not end at the token count
    assert _flags(b, qsl=qsl) & pa.CHECK_QUERY_STARTS


def test_check_query_lengths(dev):
    log("[check query lengths]")
    b = _batch(dev, False)
    assert _flags(b, max_q=b.max_query_len - 1) == pa.CHECK_QUERY_LEN
    # more new tokens than context
    ctx = b.context_lens.clone()
    ctx[1] = 10  # 77 query tokens
    assert _flags(b, ctx=ctx) == pa.CHECK_CONTEXT_SHORT
