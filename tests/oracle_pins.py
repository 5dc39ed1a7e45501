"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each pin is a function of an oracle build, so test_oracle_pins.py runs them on
the real build and test_oracle_mutants.py runs them on builds with planted
mistakes (every planted mistake must make at least one pin fail).

What pins what:
  * dense_decode_sdpa / dense_causal_sdpa: with an identity block table the
    paged result equals torch's own scaled_dot_product_attention in fp64
    (a library routine) - pins logits, scale, softmax, normalisation, the
    head grouping and the textbook causal mask.
  * golden_two_token: a hand-derived two-token example (tests/golden).
  * permutation_invariance: moving pages and remapping the table changes no
    bit - pins the page/slot gather.
  * dominant_logit, uniform_v, q_zero, single_token: closed forms.
  * split_merge: merged split partials equal the single pass for many split
    counts, including splits past the context - pins partials and merge.
  * merge_closed_form: the merge on hand-made partials.
  * gqa_equals_mha, prefill_row_equals_decode, q1_prefill_equals_decode,
    noncausal_prefill, empty_context: invariants and degenerate cases.
  * append_round_trip: after a paged append, each sequence read back by
    gathering its pages in table order shows the new rows at the end of the
    context, the prefix unchanged, and exactly one changed slot per token.
  * append_head_major_strides: a head-major pool through its strides.
  * append_hand_case: slots worked out by hand on a two-sequence example.
  * append_decode_steps_equal_chunk: token-by-token appends equal one chunk.
  * append_then_attend: append followed by attention equals torch SDPA on the
    dense context with the chunk's causal mask (pins where the chunk lands).
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from _util import DenseProblem, bits_to_f64, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _sdpa(q, k, v, scale, mask=None, is_causal=False):
    """torch fp64 SDPA for one sequence: q [n, Hq, D], k/v [L, Hq, D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=m, is_causal=is_causal, scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


def _per_row(out, T, Hq):
    return out.reshape(T, Hq, -1)


def dense_decode_sdpa(orc):
    pb = DenseProblem(seed=11, contexts=[1, 15, 16, 17, 40, 64], queries=[1] * 6,
                      Hq=4, Hkv=2, D=16, P=4)
    out, _ = orc.attention(pb.inputs)
    out = _per_row(out, 6, 4)
    G = pb.Hq // pb.Hkv
    for s in range(6):
        k = np.repeat(pb.k_dense[s], G, axis=1)
        v = np.repeat(pb.v_dense[s], G, axis=1)
        ref = _sdpa(pb.q[s:s + 1], k, v, pb.scale)
        np.testing.assert_allclose(out[s], ref[0], rtol=0, atol=1e-12)


def dense_causal_sdpa(orc):
    # the new chunk is the whole context: the textbook causal mask applies
    pb = DenseProblem(seed=12, contexts=[5, 33, 20], queries=[5, 33, 20], Hq=6, Hkv=3,
                      D=8, P=4, causal=True)
    out, _ = orc.attention(pb.inputs)
    out = _per_row(out, sum(pb.queries), pb.Hq)
    G = pb.Hq // pb.Hkv
    for s in range(3):
        a, b = pb.token_range(s)
        k = np.repeat(pb.k_dense[s], G, axis=1)
        v = np.repeat(pb.v_dense[s], G, axis=1)
        ref = _sdpa(pb.q[a:b], k, v, pb.scale, is_causal=True)
        np.testing.assert_allclose(out[a:b], ref, rtol=0, atol=1e-12)


def golden_two_token(orc):
    vals = {}
    with open(os.path.join(GOLDEN, "two_token_logistic.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *nums = line.split()
            vals[key] = [float(x) for x in nums]
    import oracle as oracle_mod
    P, D = 16, 2
    k = np.zeros((1, P, 1, D), np.float32)
    v = np.zeros((1, P, 1, D), np.float32)
    k[0, 0, 0], k[0, 1, 0] = vals["k0"], vals["k1"]
    v[0, 0, 0], v[0, 1, 0] = vals["v0"], vals["v1"]
    inp = oracle_mod.PagedInputs(
        q=f32_to_bf16_bits(np.array(vals["q"], np.float32).reshape(1, 1, D)),
        k_pool=f32_to_bf16_bits(k), v_pool=f32_to_bf16_bits(v),
        block_tables=np.zeros((1, 1), np.int32), context_lens=np.array([2], np.int32),
        query_start_loc=None, num_kv_heads=1, page_size=P, strides=(P * D, D, D),
        scale=1.0, causal=True)
    out, lse = orc.attention(inp)
    np.testing.assert_allclose(out[0], vals["out"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(lse[0], vals["lse"][0], rtol=1e-15, atol=0)


def permutation_invariance(orc):
    pb = DenseProblem(seed=13, contexts=[30, 7, 48], queries=[6, 1, 48], Hq=4, Hkv=2,
                      D=8, P=4, causal=True)
    base_out, base_lse = orc.attention(pb.inputs)
    npages = pb.k_bits.shape[0]
    rng = np.random.default_rng(99)
    extra = 5  # unused pages, poisoned with NaN
    perm = rng.permutation(npages + extra)[:npages]  # old page p -> new page perm[p]
    shape = (npages + extra,) + pb.k_bits.shape[1:]
    nan_bits = f32_to_bf16_bits(np.float32(np.nan))
    k2 = np.full(shape, nan_bits, np.uint16)
    v2 = np.full(shape, nan_bits, np.uint16)
    k2[perm] = pb.k_bits
    v2[perm] = pb.v_bits
    bt2 = np.where(pb.bt >= 0, perm[np.maximum(pb.bt, 0)], -1).astype(np.int32)
    out, lse = orc.attention(pb.make_inputs(k_bits=k2, v_bits=v2, bt=bt2))
    assert np.array_equal(out.view(np.uint64), base_out.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), base_lse.view(np.uint64))


def dominant_logit(orc):
    # q = 16 e_0 and k_t* = 16 e_0, every other k_t has k[0] = 0, scale 1:
    # z_t* = 256, z_t = 0 otherwise, so O = V_t* up to exp(-256).
    P, D, L = 4, 8, 23
    for tstar in (0, 3, 4, 11, 12, 22):
        pb = DenseProblem(seed=14 + tstar, contexts=[L], queries=[1], Hq=2, Hkv=1, D=D, P=P,
                          scale=1.0)
        qf = np.zeros((1, 2, D), np.float32)
        qf[0, :, 0] = 16.0
        k = bits_to_f64(pb.k_bits).astype(np.float32)
        flat = k.reshape(-1, 1, D)
        flat[:, 0, 0] = 0.0
        flat[tstar, 0, 0] = 16.0
        out, lse = orc.attention(pb.make_inputs(q_bits=f32_to_bf16_bits(qf),
                                                k_bits=f32_to_bf16_bits(k)))
        vstar = pb.v_dense[0][tstar, 0]
        np.testing.assert_allclose(out[0], vstar, rtol=0, atol=1e-12)
        np.testing.assert_allclose(out[1], vstar, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, 256.0, rtol=0, atol=1e-12)


def uniform_v(orc):
    pb = DenseProblem(seed=15, contexts=[19, 40], queries=[7, 1], Hq=4, Hkv=2, D=8, P=4)
    c = np.linspace(-2.0, 2.0, pb.D).astype(np.float32)  # exact in bf16? rounded below
    cb = f32_to_bf16_bits(c)
    v = np.broadcast_to(cb, pb.v_bits.shape).copy()
    out, _ = orc.attention(pb.make_inputs(v_bits=v))
    np.testing.assert_allclose(out, np.broadcast_to(bits_to_f64(cb), out.shape),
                               rtol=0, atol=1e-13)


def q_zero(orc):
    pb = DenseProblem(seed=16, contexts=[21, 9], queries=[1, 1], Hq=4, Hkv=2, D=8, P=4)
    qz = np.zeros_like(pb.q_bits)
    out, lse = orc.attention(pb.make_inputs(q_bits=qz))
    out = out.reshape(2, 4, -1)
    for s, L in enumerate([21, 9]):
        for h in range(4):
            mean = pb.v_dense[s][:, h // 2].mean(axis=0)
            np.testing.assert_allclose(out[s, h], mean, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse.reshape(2, 4), np.log([[21.0] * 4, [9.0] * 4]),
                               rtol=0, atol=1e-13)
    # causal chunk with no prefix: row i sees tokens 0..i
    pb = DenseProblem(seed=17, contexts=[10], queries=[10], Hq=2, Hkv=1, D=4, P=4)
    out, lse = orc.attention(pb.make_inputs(q_bits=np.zeros_like(pb.q_bits)))
    out = out.reshape(10, 2, -1)
    for i in range(10):
        np.testing.assert_allclose(out[i, 0], pb.v_dense[0][: i + 1, 0].mean(axis=0),
                                   rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse.reshape(10, 2)[:, 0], np.log(np.arange(1, 11.0)),
                               rtol=0, atol=1e-13)


def single_token(orc):
    pb = DenseProblem(seed=18, contexts=[1], queries=[1], Hq=4, Hkv=4, D=16, P=16)
    out, lse = orc.attention(pb.inputs)
    for h in range(4):
        np.testing.assert_array_equal(out[h], pb.v_dense[0][0, h])
        z0 = pb.scale * float(np.dot(pb.q[0, h], pb.k_dense[0][0, h]))
        np.testing.assert_allclose(lse[h], z0, rtol=1e-14, atol=1e-14)


def split_merge(orc):
    cases = [
        DenseProblem(seed=19, contexts=[100, 37, 1, 64], queries=[1] * 4, Hq=4, Hkv=2, D=8,
                     P=4),
        DenseProblem(seed=20, contexts=[50, 29], queries=[13, 29], Hq=4, Hkv=1, D=8, P=4,
                     causal=True),
    ]
    for pb in cases:
        single, single_lse = orc.attention(pb.inputs)
        Lmax = max(pb.contexts)
        for S in (1, 2, 3, 7, 8, 16, 64):
            pages = -(-Lmax // pb.P)
            split_tokens = -(-pages // S) * pb.P  # page-aligned, covers Lmax
            po, pl = orc.partials(pb.inputs, split_tokens, S)
            out, lse = orc.merge(po, pl)
            np.testing.assert_allclose(out, single, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, single_lse, rtol=1e-13, atol=1e-13)
        # splits of one token each: every split is a single (or no) token
        S1 = Lmax
        po, pl = orc.partials(pb.inputs, 1, S1)
        out, lse = orc.merge(po, pl)
        np.testing.assert_allclose(out, single, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, single_lse, rtol=1e-13, atol=1e-13)


def merge_closed_form(orc):
    D = 5
    o1 = np.arange(D, dtype=np.float64)
    o2 = np.arange(D, dtype=np.float64)[::-1].copy()
    po = np.stack([o1, o2, np.zeros(D)])[None]
    pl = np.array([[0.0, math.log(3.0), -math.inf]])
    out, lse = orc.merge(po, pl)
    np.testing.assert_allclose(out[0], (o1 + 3 * o2) / 4, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(4.0), rtol=1e-15)
    # a single finite partial passes through unchanged
    pl = np.array([[-math.inf, 2.5, -math.inf]])
    out, lse = orc.merge(po, pl)
    np.testing.assert_allclose(out[0], o2, rtol=0, atol=0)
    assert lse[0] == 2.5
    # every partial empty: O = 0, LSE = -inf
    pl = np.full((1, 3), -math.inf)
    out, lse = orc.merge(po, pl)
    assert np.all(out == 0) and lse[0] == -math.inf


def gqa_equals_mha(orc):
    pb = DenseProblem(seed=21, contexts=[33, 17], queries=[5, 1], Hq=8, Hkv=2, D=8, P=4)
    out, lse = orc.attention(pb.inputs)
    G = pb.Hq // pb.Hkv
    k_rep = np.repeat(pb.k_bits, G, axis=2)  # head h of the copy holds KV head h // G
    v_rep = np.repeat(pb.v_bits, G, axis=2)
    out2, lse2 = orc.attention(pb.make_inputs(k_bits=k_rep, v_bits=v_rep, Hkv=pb.Hq))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def prefill_row_equals_decode(orc):
    L, q = 37, 9
    pb = DenseProblem(seed=22, contexts=[L], queries=[q], Hq=4, Hkv=2, D=8, P=4, causal=True)
    out, lse = orc.attention(pb.inputs)
    out = out.reshape(q, 4, -1)
    lse = lse.reshape(q, 4)
    for i in range(q):
        d_inp = pb.make_inputs(q_bits=pb.q_bits[i:i + 1], contexts=[L - q + i + 1], qsl=None)
        o, l = orc.attention(d_inp)
        assert np.array_equal(out[i], o) and np.array_equal(lse[i], l)


def q1_prefill_equals_decode(orc):
    pb = DenseProblem(seed=23, contexts=[12, 40, 3], queries=[1, 1, 1], Hq=4, Hkv=2, D=8,
                      P=4, decode_layout=True)
    out, lse = orc.attention(pb.inputs)
    qsl = np.array([0, 1, 2, 3], np.int32)
    out2, lse2 = orc.attention(pb.make_inputs(qsl=qsl, causal=True))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def noncausal_prefill(orc):
    L, q = 26, 6
    pb = DenseProblem(seed=24, contexts=[L], queries=[q], Hq=2, Hkv=1, D=8, P=4,
                      causal=False)
    out, _ = orc.attention(pb.inputs)
    out = out.reshape(q, 2, -1)
    for i in range(q):
        o, _ = orc.attention(pb.make_inputs(q_bits=pb.q_bits[i:i + 1], qsl=None))
        assert np.array_equal(out[i], o)
    k = np.repeat(pb.k_dense[0], 2, axis=1)
    v = np.repeat(pb.v_dense[0], 2, axis=1)
    ref = _sdpa(pb.q, k, v, pb.scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def empty_context(orc):
    pb = DenseProblem(seed=25, contexts=[0, 5], queries=[1, 1], Hq=2, Hkv=1, D=4, P=4)
    out, lse = orc.attention(pb.inputs)
    assert np.all(out[:2] == 0) and np.all(lse[:2] == -math.inf)
    assert np.all(np.isfinite(out[2:])) and np.all(np.isfinite(lse[2:]))


def _append(orc, *args, **kw):
    """The append oracle; a refused write (out-of-range position) fails the pin."""
    try:
        return orc.append(*args, **kw)
    except RuntimeError as e:
        raise AssertionError(str(e))


def _random_bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _append_case(seed, P=4, Hkv=2, D=8, spare=3):
    """Shuffled pages, mixed chunk lengths: a chunk crossing pages, a chunk that
    is the whole context, a decode-like single token, an empty chunk, and a
    chunk ending exactly on a page boundary."""
    rng = np.random.default_rng(seed)
    contexts = [7, 4, 13, 9, 8]
    queries = [3, 4, 1, 0, 4]
    blocks = [-(-c // P) for c in contexts]
    npages = sum(blocks) + spare
    order = rng.permutation(npages)
    bt = np.full((len(contexts), max(blocks) + 1), 0, np.int32)
    base = 0
    for s, n in enumerate(blocks):
        bt[s, :n] = order[base:base + n]
        base += n
    qsl = np.concatenate([[0], np.cumsum(queries)]).astype(np.int32)
    return dict(rng=rng, P=P, Hkv=Hkv, D=D, npages=npages, bt=bt, contexts=contexts,
                queries=queries, qsl=qsl, T=int(qsl[-1]))


def _seq_view(pool, bt_row, nblocks, L):
    """Logical rows [0, L) of one sequence of a [pages, P, Hkv, D] pool, by
    gathering its pages in table order and flattening (page, slot)."""
    return pool[bt_row[:nblocks]].reshape((-1,) + pool.shape[2:])[:L]


def append_round_trip(orc):
    c = _append_case(31)
    P, Hkv, D, rng = c["P"], c["Hkv"], c["D"], c["rng"]
    shape = (c["npages"], P, Hkv, D)
    k0, v0 = _random_bits(rng, shape), _random_bits(rng, shape)
    kn, vn = _random_bits(rng, (c["T"], Hkv, D)), _random_bits(rng, (c["T"], Hkv, D))
    k1, v1 = _append(orc, k0, v0, P, (P * Hkv * D, Hkv * D, D), kn, vn, c["bt"],
                     c["contexts"], c["qsl"])
    for s, (L, q) in enumerate(zip(c["contexts"], c["queries"])):
        nb = -(-L // P)
        a, b = c["qsl"][s], c["qsl"][s + 1]
        for pool1, pool0, new in ((k1, k0, kn), (v1, v0, vn)):
            seq1 = _seq_view(pool1, c["bt"][s], nb, L)
            seq0 = _seq_view(pool0, c["bt"][s], nb, L)
            assert np.array_equal(seq1[L - q:], new[a:b])     # new rows at the context end
            assert np.array_equal(seq1[:L - q], seq0[:L - q])  # the prefix is untouched
    # nothing else moved: exactly one (page, slot) per new token changed
    for pool1, pool0 in ((k1, k0), (v1, v0)):
        changed = (pool1 != pool0).any(axis=(2, 3))
        assert int(changed.sum()) == c["T"]


def append_head_major_strides(orc):
    """A pool laid out (page, kv head, slot, d) through its strides gives the
    same rows as the default (page, slot, kv head, d) layout."""
    c = _append_case(32)
    P, Hkv, D, rng = c["P"], c["Hkv"], c["D"], c["rng"]
    k0, v0 = _random_bits(rng, (c["npages"], P, Hkv, D)), _random_bits(rng, (c["npages"], P, Hkv, D))
    kn, vn = _random_bits(rng, (c["T"], Hkv, D)), _random_bits(rng, (c["T"], Hkv, D))
    args = (kn, vn, c["bt"], c["contexts"], c["qsl"])
    k1, v1 = _append(orc, k0, v0, P, (P * Hkv * D, Hkv * D, D), *args)
    kh = np.ascontiguousarray(k0.transpose(0, 2, 1, 3))
    vh = np.ascontiguousarray(v0.transpose(0, 2, 1, 3))
    k2, v2 = _append(orc, kh, vh, P, (Hkv * P * D, D, P * D), *args)
    assert np.array_equal(k2.transpose(0, 2, 1, 3), k1)
    assert np.array_equal(v2.transpose(0, 2, 1, 3), v1)


def append_hand_case(orc):
    """P = 4, one kv head, D = 2.  Sequence 0 holds 6 tokens, the last 3 new,
    through table row [2, 0]: positions 3, 4, 5 are page 2 slot 3, page 0 slot
    0, page 0 slot 1.  Sequence 1 holds 1 token, new, through [1, 1]: position
    0 is page 1 slot 0."""
    P, D = 4, 2
    k0 = np.zeros((3, P, 1, D), np.uint16)
    v0 = np.full((3, P, 1, D), 7, np.uint16)
    kn = np.array([[[11, 12]], [[21, 22]], [[31, 32]], [[41, 42]]], np.uint16)
    vn = kn + 100
    k1, v1 = _append(orc, k0, v0, P, (P * D, D, D), kn, vn,
                     np.array([[2, 0], [1, 1]], np.int32), [6, 1],
                     np.array([0, 3, 4], np.int32))
    want_k, want_v = k0.copy(), v0.copy()
    for (page, slot), row in {(2, 3): 0, (0, 0): 1, (0, 1): 2, (1, 0): 3}.items():
        want_k[page, slot, 0] = kn[row, 0]
        want_v[page, slot, 0] = vn[row, 0]
    assert np.array_equal(k1, want_k) and np.array_equal(v1, want_v)


def append_decode_steps_equal_chunk(orc):
    """Appending a chunk token by token (one-token-per-sequence layout, the
    context growing by one each step) fills the same slots as one chunk."""
    c = _append_case(33)
    P, Hkv, D, rng = c["P"], c["Hkv"], c["D"], c["rng"]
    strides = (P * Hkv * D, Hkv * D, D)
    k0, v0 = _random_bits(rng, (c["npages"], P, Hkv, D)), _random_bits(rng, (c["npages"], P, Hkv, D))
    kn, vn = _random_bits(rng, (c["T"], Hkv, D)), _random_bits(rng, (c["T"], Hkv, D))
    k1, v1 = _append(orc, k0, v0, P, strides, kn, vn, c["bt"], c["contexts"], c["qsl"])
    ks, vs = k0, v0
    qmax = max(c["queries"])
    for step in range(qmax):
        # every sequence still adding tokens gets its next one; the others re-append
        # their last prefix row unchanged (a no-op write of the value already there)
        rows_k, rows_v, lens = [], [], []
        for s, (L, q) in enumerate(zip(c["contexts"], c["queries"])):
            if step < q:
                r = c["qsl"][s] + step
                rows_k.append(kn[r])
                rows_v.append(vn[r])
                lens.append(L - q + step + 1)
            else:
                lens.append(0)  # context shorter than its one token: nothing written
                rows_k.append(np.zeros((Hkv, D), np.uint16))
                rows_v.append(np.zeros((Hkv, D), np.uint16))
        ks, vs = _append(orc, ks, vs, P, strides, np.stack(rows_k), np.stack(rows_v), c["bt"],
                         lens, None)
    assert np.array_equal(ks, k1) and np.array_equal(vs, v1)


def append_then_attend(orc):
    """Append a chunk, then attend: equals torch SDPA over the dense context
    (cached prefix followed by the new rows) with the chunk's causal mask."""
    import oracle as oracle_mod
    P, Hq, Hkv, D = 4, 4, 2, 8
    L, q = 23, 7
    rng = np.random.default_rng(34)
    npages = -(-L // P) + 2
    bt = rng.permutation(npages)[None, :].astype(np.int32)
    shape = (npages, P, Hkv, D)
    k0, v0 = _random_bits(rng, shape), _random_bits(rng, shape)
    kn, vn = _random_bits(rng, (q, Hkv, D)), _random_bits(rng, (q, Hkv, D))
    qb = _random_bits(rng, (q, Hq, D))
    strides = (P * Hkv * D, Hkv * D, D)
    qsl = np.array([0, q], np.int32)
    k1, v1 = _append(orc, k0, v0, P, strides, kn, vn, bt, [L], qsl)
    inp = oracle_mod.PagedInputs(q=qb, k_pool=k1, v_pool=v1, block_tables=bt,
                                 context_lens=np.array([L], np.int32), query_start_loc=qsl,
                                 num_kv_heads=Hkv, page_size=P, strides=strides,
                                 scale=0.25, causal=True)
    out, _ = orc.attention(inp)
    nb = -(-L // P)
    kd = np.concatenate([bits_to_f64(_seq_view(k0, bt[0], nb, L)[:L - q]), bits_to_f64(kn)])
    vd = np.concatenate([bits_to_f64(_seq_view(v0, bt[0], nb, L)[:L - q]), bits_to_f64(vn)])
    G = Hq // Hkv
    mask = np.tril(np.ones((q, L), bool), k=L - q)
    ref = _sdpa(bits_to_f64(qb), np.repeat(kd, G, axis=1), np.repeat(vd, G, axis=1), 0.25,
                mask=mask)
    np.testing.assert_allclose(out.reshape(q, Hq, D), ref, rtol=0, atol=1e-12)


APPEND_PINS = [append_round_trip, append_head_major_strides, append_hand_case,
               append_decode_steps_equal_chunk, append_then_attend]

ALL_PINS = [dense_decode_sdpa, dense_causal_sdpa, golden_two_token, permutation_invariance,
            dominant_logit, uniform_v, q_zero, single_token, split_merge, merge_closed_form,
            gqa_equals_mha, prefill_row_equals_decode, q1_prefill_equals_decode,
            noncausal_prefill, empty_context] + APPEND_PINS
