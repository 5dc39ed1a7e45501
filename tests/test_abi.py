"""The C-ABI library on the CPU: it loads, exports every symbol include/pa.h
declares, and its host-side checks reject bad arguments before any launch
(no compute call is made here)."""
import ctypes
import os
import re

import pytest

from paged_gqa_attention_pa_amd import pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.library_path()):
        pytest.skip("libpa.so not built (run __graft_entry__.build())")
    return pa.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(declared) == set(pa.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def _problem(**kw):
    pb = pa.Problem()
    vals = dict(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                max_blocks_per_seq=512, kv_stride_page=16 * 8 * 128, kv_stride_token=8 * 128,
                kv_stride_head=128, max_context_len=8192, max_query_len=1,
                total_query_tokens=4, causal=1, scale=0.08838834764831845,
                out_dtype=pa.PA_BF16)
    vals.update(kw)
    for k, v in vals.items():
        setattr(pb, k, v)
    return pb


def _select(lib, pb):
    t = pa.Tiles()
    ws = ctypes.c_size_t(0)
    st = lib.pa_select_tiles(ctypes.byref(pb), ctypes.byref(t), ctypes.byref(ws))
    return st, t, ws.value


def test_select_tiles_decode_and_prefill(lib):
    st, t, ws = _select(lib, _problem())
    assert st == pa.PA_OK and t.num_splits >= 1 and t.kv_tile == 16
    if t.num_splits > 1:
        assert ws >= 4 * 32 * t.num_splits * 129 * 4
    # long context, batch 1: split-KV engages
    st, t, ws = _select(lib, _problem(num_seqs=1, total_query_tokens=1, max_context_len=32768,
                                      max_blocks_per_seq=2048))
    assert st == pa.PA_OK and t.num_splits > 8 and ws > 0
    st, t, ws = _select(lib, _problem(max_query_len=2048, total_query_tokens=8192,
                                      max_context_len=3072))
    assert st == pa.PA_OK and t.q_tokens_per_tile == 64 and t.num_splits == 1 and ws == 0
    assert t.tile_splits == 1
    # two long-prefix chunks alone: tiles are split, and the workspace holds
    # their partials (fp32 [T*Hq, ts, 128] + lse)
    T = 2 * 512
    st, t, ws = _select(lib, _problem(num_seqs=2, max_query_len=512, total_query_tokens=T,
                                      max_context_len=4608, max_blocks_per_seq=512))
    assert st == pa.PA_OK and t.tile_splits > 1 and t.num_splits == 1
    assert ws >= T * 32 * t.tile_splits * 129 * 4
    # the same chunks beside decode rows: decode splits, no tile split
    st, t, ws = _select(lib, _problem(num_seqs=18, max_query_len=512, total_query_tokens=T + 16,
                                      max_context_len=16384, max_blocks_per_seq=1024))
    assert st == pa.PA_OK and t.tile_splits == 1 and t.num_splits > 1
    # where single-token sequences are query tiles of their own (head dims 64
    # and 256, G = 16), their key runs are split: about 32 * head_dim keys a
    # run, at most eight workgroups per CU in all
    mixed = dict(num_seqs=18, max_query_len=512, total_query_tokens=T + 16,
                 max_context_len=16384, max_blocks_per_seq=1024)
    for kw, want in ((dict(head_dim=64, kv_stride_page=16 * 8 * 64, kv_stride_token=8 * 64,
                           kv_stride_head=64), 7),
                     (dict(num_q_heads=64, num_kv_heads=4, kv_stride_page=16 * 4 * 128,
                           kv_stride_token=4 * 128), 4),
                     (dict(head_dim=256, kv_stride_page=16 * 8 * 256, kv_stride_token=8 * 256,
                           kv_stride_head=256), 2)):
        st, t, ws = _select(lib, _problem(**mixed, **kw))
        assert st == pa.PA_OK and t.tile_splits == want, (kw, t.tile_splits)
        D = kw.get("head_dim", 128)
        Hq = kw.get("num_q_heads", 32)
        assert ws >= (T + 16) * Hq * t.tile_splits * (D + 1) * 4
    # a mixed batch that already fills the chip (far more than eight query
    # tiles per CU) keeps its tiles whole
    st, t, ws = _select(lib, _problem(num_seqs=200, max_query_len=2048, total_query_tokens=200000,
                                      max_context_len=16384, max_blocks_per_seq=1024,
                                      head_dim=64, kv_stride_page=16 * 8 * 64,
                                      kv_stride_token=8 * 64, kv_stride_head=64))
    assert st == pa.PA_OK and t.tile_splits == 1


@pytest.mark.parametrize("field,value,status", [
    ("num_q_heads", 30, pa.PA_ERR_INVALID_ARG),       # Hq % Hkv != 0
    ("head_dim", 96, pa.PA_ERR_UNSUPPORTED),
    ("page_size", 12, pa.PA_ERR_INVALID_ARG),         # not a power of two
    ("page_size", 0, pa.PA_ERR_INVALID_ARG),
    ("kv_stride_token", 1020, pa.PA_ERR_INVALID_ARG),  # not a multiple of 8
    # a page's slots span 2^31 elements or more
    ("kv_stride_token", 1 << 27, pa.PA_ERR_UNSUPPORTED),
    ("max_context_len", 512 * 16 + 1, pa.PA_ERR_INVALID_ARG),
    ("num_seqs", -1, pa.PA_ERR_INVALID_ARG),
    ("out_dtype", 7, pa.PA_ERR_INVALID_ARG),
    ("causal", 2, pa.PA_ERR_INVALID_ARG),
    ("scale", float("nan"), pa.PA_ERR_INVALID_ARG),
    ("scale", 0.0, pa.PA_ERR_INVALID_ARG),
    ("scale", -0.5, pa.PA_ERR_INVALID_ARG),
    ("scale", float("inf"), pa.PA_ERR_INVALID_ARG),
])
def test_select_tiles_rejects(lib, field, value, status):
    st, _, _ = _select(lib, _problem(**{field: value}))
    assert st == status


@pytest.mark.parametrize("page_size", [16, 32, 64, 128, 256, 1024])
def test_page_sizes_accepted(lib, page_size):
    """Pages of any power of two from 16 slots: a page is 2^k 16-key tiles."""
    st, t, ws = _select(lib, _problem(page_size=page_size, kv_stride_page=page_size * 8 * 128))
    assert st == pa.PA_OK and t.num_splits >= 1 and ws > 0


def test_page_size_below_one_tile(lib):
    st, _, _ = _select(lib, _problem(page_size=8, max_blocks_per_seq=1024))
    assert st == pa.PA_ERR_UNSUPPORTED


def test_page_tile_index_bound(lib):
    """16-key tile indices of a table row (max_blocks_per_seq * P / 16) must fit in int."""
    big = dict(page_size=1024, kv_stride_page=1024 * 8 * 128)
    st, _, _ = _select(lib, _problem(max_blocks_per_seq=(1 << 31) // 64 - 1, **big))
    assert st == pa.PA_OK
    st, _, _ = _select(lib, _problem(max_blocks_per_seq=(1 << 31) // 64, **big))
    assert st == pa.PA_ERR_UNSUPPORTED


def test_group_sizes_built(lib):
    for hq, hkv in [(8, 8), (16, 8), (32, 8), (64, 8), (16, 1), (32, 1)]:
        st, t, _ = _select(lib, _problem(num_q_heads=hq, num_kv_heads=hkv))
        assert st == pa.PA_OK, (hq, hkv)
    st, _, _ = _select(lib, _problem(num_q_heads=64, num_kv_heads=1))  # G = 64
    assert st == pa.PA_ERR_UNSUPPORTED


def test_head_dims_built(lib):
    """Head dims 64, 128 and 256 are built for decode, short query runs and
    query tiles; the query tile is 256 rows (256 / G tokens, 8 wavefronts),
    128 rows at head dim 256 (4 wavefronts)."""
    for d in (64, 128, 256):
        kw = dict(head_dim=d, kv_stride_page=16 * 8 * d, kv_stride_token=8 * d, kv_stride_head=d)
        st, t, ws = _select(lib, _problem(**kw))  # decode
        assert st == pa.PA_OK, d
        st, t, ws = _select(lib, _problem(max_query_len=4, total_query_tokens=16, **kw))
        assert st == pa.PA_OK, d
        st, t, _ = _select(lib, _problem(max_query_len=64, total_query_tokens=256, **kw))
        assert st == pa.PA_OK, d
        assert t.q_tokens_per_tile == (32 if d == 256 else 64), d
        assert t.waves_per_wg == (4 if d == 256 else 8), d
    # 16 rows x 256 dims per row block: at most two row blocks, longer runs
    # take the query tiles
    kw = dict(head_dim=256, kv_stride_page=16 * 8 * 256, kv_stride_token=8 * 256,
              kv_stride_head=256)
    st, t, _ = _select(lib, _problem(max_query_len=8, total_query_tokens=32, **kw))
    assert st == pa.PA_OK and t.kv_tile == 16
    st, t, _ = _select(lib, _problem(max_query_len=9, total_query_tokens=36, **kw))
    assert st == pa.PA_OK and t.kv_tile == 32 and t.q_tokens_per_tile == 32


def test_select_tiles_short_runs(lib):
    """Short query runs (2 <= max_query_len, max_query_len * G <= 64) and
    decode at G = 32 take one Q-block per (sequence, kv head) unit on the
    even-work grid, with a workspace of S + 1 slots per (token, head) row."""
    cases = [dict(max_query_len=4, total_query_tokens=16),           # G = 4, 16 rows
             dict(max_query_len=16, total_query_tokens=64),          # G = 4, 64 rows
             dict(num_q_heads=32, num_kv_heads=1, max_query_len=1),  # G = 32 decode
             dict(num_q_heads=32, num_kv_heads=1, max_query_len=2, total_query_tokens=8)]
    for kw in cases:
        pb = _problem(**kw)
        st, t, ws = _select(lib, pb)
        assert st == pa.PA_OK, kw
        assert t.kv_tile == 16 and t.waves_per_wg == 4 and (t.variant & 6) == 6, kw
        rows = pb.total_query_tokens * pb.num_q_heads if pb.max_query_len > 1 \
            else pb.num_seqs * pb.num_q_heads
        assert ws >= rows * (t.num_splits + 1) * 129 * 4, kw
    # 17 tokens x 4 heads = 68 rows: the query tiles
    st, t, _ = _select(lib, _problem(max_query_len=17, total_query_tokens=68))
    assert st == pa.PA_OK and t.kv_tile == 32


def test_short_run_decode_variant_workspace(lib):
    """Variant bit 3 moves decode rows (G <= 16) to the short-run kernel: the
    table never sets it, and with it the workspace is needed even at S = 1
    (S + 1 slots per row plus the piece counts)."""
    pb = _problem()
    st, t, _ = _select(lib, pb)
    assert st == pa.PA_OK and (t.variant & 8) == 0
    for S in (1, 4):
        t1 = pa.Tiles(16, S, 4, 1, 14)
        ws = ctypes.c_size_t(0)
        assert lib.pa_workspace_size(ctypes.byref(pb), ctypes.byref(t1), ctypes.byref(ws)) == pa.PA_OK
        assert ws.value >= pb.num_seqs * pb.num_q_heads * (S + 1) * 129 * 4
        fake = ctypes.c_void_p(0x10000)  # never dereferenced: the workspace check fails first
        assert lib.pa_decode(ctypes.byref(pb), ctypes.byref(t1), fake, fake, fake, fake, fake,
                             fake, None, None, 0, None) == pa.PA_ERR_WORKSPACE


def _gen_table(name):
    """A constexpr array of the generated tile-table header, as nested lists."""
    src = open(os.path.join(os.path.dirname(pa.__file__), "csrc", "pa_tile_table_gen.h")).read()
    body = re.search(name + r"(?:\[\d*\])*\s*=\s*\{(.*?)\};", src, re.S).group(1)
    rows = re.findall(r"\{([^{}]*)\}", body)
    if not rows:
        return [int(x) for x in body.split(",") if x.strip()]
    return [[int(x) for x in r.split(",") if x.strip()] for r in rows]


def test_short_run_split_table(lib):
    """Short query runs take their split bound from the short-run table of
    the generated header, by (head dim, G >= 16) key and (units rounded
    down, context bound rounded up); unswept buckets keep the decode choice."""
    units_b = _gen_table("kShortUnitBuckets")
    ctx_b = _gen_table("kShortCtxBuckets")
    keys = _gen_table("kShortKeys")
    flat = _gen_table("kShortSplits")
    assert len(flat) == len(keys) * len(units_b) and all(len(r) == len(ctx_b) for r in flat)
    table = {tuple(k): flat[i * len(units_b):(i + 1) * len(units_b)] for i, k in enumerate(keys)}
    checked = 0
    for i, units in enumerate(units_b):
        for j, ctx in enumerate(ctx_b):
            blocks = -(-ctx // 16)
            shapes = [((128, 1), dict(num_q_heads=32, num_kv_heads=1, num_seqs=units,
                                      total_query_tokens=units))]           # G = 32 decode
            if units >= 8:                                                  # G = 4, 4 tokens
                shapes.append(((128, 0), dict(num_seqs=units // 8, max_query_len=4,
                                              total_query_tokens=units // 2)))
            for key, kw in shapes:
                want = table[key][i][j]
                pb = _problem(max_context_len=ctx, max_blocks_per_seq=blocks, **kw)
                st, t, _ = _select(lib, pb)
                assert st == pa.PA_OK, kw
                if want > 0:
                    assert t.num_splits == want, (units, ctx, kw)
                    checked += 1
                # one unit more than the bucket, same context: same bucket
                kw2 = dict(kw, num_seqs=kw["num_seqs"] + 1,
                           total_query_tokens=kw["total_query_tokens"] + 1)
                st, t2, _ = _select(lib, _problem(max_context_len=ctx, max_blocks_per_seq=blocks,
                                                  **kw2))
                next_floor = i + 1 < len(units_b) and (
                    (kw2["num_seqs"] * kw2.get("num_kv_heads", 8)) >= units_b[i + 1])
                if want > 0 and not next_floor:
                    assert t2.num_splits == want, (units, ctx, kw2)
    assert checked > 0


def test_compute_calls_reject_before_launch(lib):
    pb = _problem()
    t = pa.Tiles(16, 1, 4, 1, 0)
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: checks fail first
    nul = None
    # null q
    assert lib.pa_decode(ctypes.byref(pb), ctypes.byref(t), nul, fake, fake, fake, fake, fake,
                         nul, nul, 0, nul) == pa.PA_ERR_INVALID_ARG
    # misaligned q
    mis = ctypes.c_void_p(0x10008)
    assert lib.pa_decode(ctypes.byref(pb), ctypes.byref(t), mis, fake, fake, fake, fake, fake,
                         nul, nul, 0, nul) == pa.PA_ERR_INVALID_ARG
    # split-KV without workspace
    t2 = pa.Tiles(16, 8, 4, 1, 0)
    assert lib.pa_decode(ctypes.byref(pb), ctypes.byref(t2), fake, fake, fake, fake, fake, fake,
                         nul, nul, 0, nul) == pa.PA_ERR_WORKSPACE
    # even-work grid without the separate merge
    t5 = pa.Tiles(16, 8, 4, 1, 4)
    assert lib.pa_decode(ctypes.byref(pb), ctypes.byref(t5), fake, fake, fake, fake, fake, fake,
                         nul, fake, 1 << 30, nul) == pa.PA_ERR_INVALID_ARG
    # too many splits
    t3 = pa.Tiles(16, 100000, 4, 1, 0)
    assert lib.pa_decode(ctypes.byref(pb), ctypes.byref(t3), fake, fake, fake, fake, fake, fake,
                         nul, nul, 0, nul) == pa.PA_ERR_INVALID_ARG
    # split query tiles without the workspace for their partials
    pt = _problem(max_query_len=64, total_query_tokens=256)
    t4 = pa.Tiles(32, 1, 8, 64, 0, 2)
    assert lib.pa_prefill(ctypes.byref(pt), ctypes.byref(t4), fake, fake, fake, fake, fake, fake,
                          fake, nul, nul, 0, nul) == pa.PA_ERR_WORKSPACE
    # a decode call given a problem with longer query runs
    pq = _problem(max_query_len=4, total_query_tokens=16)
    assert lib.pa_decode(ctypes.byref(pq), ctypes.byref(t), fake, fake, fake, fake, fake, fake,
                         nul, nul, 0, nul) == pa.PA_ERR_INVALID_ARG
    # prefill without query_start_loc
    pp = _problem(max_query_len=64, total_query_tokens=256)
    assert lib.pa_prefill(ctypes.byref(pp), ctypes.byref(t), fake, nul, fake, fake, fake, fake,
                          fake, nul, nul, 0, nul) == pa.PA_ERR_INVALID_ARG
    # reduce: bad head_dim, bad dtype
    assert lib.pa_splitkv_reduce(fake, fake, 4, 2, 126, fake, pa.PA_FP32, nul, nul) == \
        pa.PA_ERR_INVALID_ARG
    assert lib.pa_splitkv_reduce(fake, fake, 4, 2, 128, fake, 9, nul, nul) == \
        pa.PA_ERR_INVALID_ARG
    # empty batches are a no-op that launches nothing
    assert lib.pa_decode(ctypes.byref(_problem(num_seqs=0, total_query_tokens=0)),
                         ctypes.byref(t), fake, fake, fake, fake, fake, fake, nul, nul, 0,
                         nul) == pa.PA_OK
    assert lib.pa_splitkv_reduce(fake, fake, 0, 2, 128, fake, pa.PA_FP32, nul, nul) == pa.PA_OK


def test_cache_append_rejects_before_launch(lib):
    fake = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10008)
    nul = None

    def call(pb, k_new=fake, v_new=fake, qsl=nul, bt=fake, cl=fake, kp=fake, vp=fake):
        return lib.pa_cache_append(ctypes.byref(pb), k_new, v_new, qsl, bt, cl, kp, vp, nul)

    pb = _problem()
    assert call(pb, k_new=nul) == pa.PA_ERR_INVALID_ARG
    assert call(pb, vp=nul) == pa.PA_ERR_INVALID_ARG
    assert call(pb, bt=nul) == pa.PA_ERR_INVALID_ARG
    assert call(pb, v_new=mis) == pa.PA_ERR_INVALID_ARG
    assert call(pb, kp=mis) == pa.PA_ERR_INVALID_ARG
    # one token per sequence unless query_start_loc is given
    assert call(_problem(total_query_tokens=9)) == pa.PA_ERR_INVALID_ARG
    assert call(_problem(head_dim=96, kv_stride_head=96)) == pa.PA_ERR_UNSUPPORTED
    assert call(_problem(page_size=8, max_blocks_per_seq=1024)) == pa.PA_ERR_UNSUPPORTED
    assert call(_problem(kv_stride_token=12)) == pa.PA_ERR_INVALID_ARG
    # nothing to write: no launch
    assert call(_problem(num_seqs=0, total_query_tokens=0)) == pa.PA_OK
    assert call(_problem(total_query_tokens=0), qsl=fake) == pa.PA_OK


def test_check_inputs_rejects_before_launch(lib):
    """pa_check_inputs validates its host arguments before enqueuing."""
    pb = _problem()
    fake = ctypes.c_void_p(0x10000)
    nul = None
    assert lib.pa_check_inputs(ctypes.byref(pb), 64, nul, fake, nul, fake, nul) == \
        pa.PA_ERR_INVALID_ARG  # no block table
    assert lib.pa_check_inputs(ctypes.byref(pb), 64, fake, fake, nul, nul, nul) == \
        pa.PA_ERR_INVALID_ARG  # no flags word
    assert lib.pa_check_inputs(ctypes.byref(pb), 0, fake, fake, nul, fake, nul) == \
        pa.PA_ERR_INVALID_ARG  # empty pool
    pp = _problem(max_query_len=64, total_query_tokens=256)
    assert lib.pa_check_inputs(ctypes.byref(pp), 64, fake, fake, nul, fake, nul) == \
        pa.PA_ERR_INVALID_ARG  # several tokens per sequence without query_start_loc


def test_status_strings(lib):
    for s in range(5):
        assert pa.status_string(s)
    assert "workspace" in pa.status_string(pa.PA_ERR_WORKSPACE)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without a built libpa.so every entry point raises: there is no
    fallback path that would compute anything elsewhere."""
    import torch
    monkeypatch.setattr(pa, "_lib", None)
    monkeypatch.setattr(pa, "_LIB_PATH", str(tmp_path / "libpa.so"))
    with pytest.raises(ImportError):
        pa.load()
    t = torch.zeros((1, 32, 128), dtype=torch.bfloat16)
    pool = torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16)
    bt = torch.zeros((1, 4), dtype=torch.int32)
    ctx = torch.ones(1, dtype=torch.int32)
    with pytest.raises(ImportError):
        pa.decode(t, pool, pool, bt, ctx, 0.088, 16)
    with pytest.raises(ImportError):
        pa.prefill(t, torch.tensor([0, 1], dtype=torch.int32), pool, pool, bt, ctx, 0.088, 16, 1)


def test_product_code_never_imports_the_oracle():
    """Only the tests, the smoke check and the benchmark's CPU baseline may
    reach the oracle; the package (binding, build, tuning) must not."""
    pkg = os.path.join(ROOT, "paged_gqa_attention_pa_amd")
    offenders = []
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                if re.search(r"^\s*(import|from)\s+oracle\b|pa_oracle|liboracle", text, re.M):
                    offenders.append(os.path.join(dirpath, f))
    assert not offenders, offenders
