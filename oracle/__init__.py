"""Python loader for the fp64 paged-attention oracle (pa_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The oracle shares no code with the
HIP library and never imports it.

Inputs are plain host numpy arrays: bf16 values as their uint16 bit
patterns, int32 tables.  Results are fp64.  What the C code computes, with the
passages of the pages it follows, is stated in the header of pa_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_default = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB, flags=("-O2",)) -> str:
    """Compile the oracle with gcc (plain C, -O2, pthreads); `flags` replaces
    the optimisation flags (e.g. a sanitizer build)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc"] + list(flags) + ["-std=c99", "-D_POSIX_C_SOURCE=200809L",
                                                       "-Wall", "-shared", "-fPIC", "-pthread",
                                                       src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, lib_path: str = _LIB):
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        common = [i32, i32, i32, i32, i32, P, P, P, P, i64, i64, i64, P, i32, P, f32, i32]
        lib.pa_oracle_attention.argtypes = common + [P, i64, P, P, i32]
        lib.pa_oracle_attention.restype = ctypes.c_int
        lib.pa_oracle_partials.argtypes = common + [i32, i32, P, i64, P, P, i32]
        lib.pa_oracle_partials.restype = ctypes.c_int
        lib.pa_oracle_merge.argtypes = [P, P, i64, i32, i32, P, P]
        lib.pa_oracle_merge.restype = ctypes.c_int
        lib.pa_oracle_append.argtypes = [i32, i32, i32, i32, P, P, P, P, P, i64, i64, i64, i64,
                                         P, i32, P]
        lib.pa_oracle_append.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def attention(self, inp, rows=None, threads=None):
        return _attention(self.lib, inp, rows, threads)

    def partials(self, inp, split_tokens, num_splits, rows=None, threads=None):
        return _partials(self.lib, inp, split_tokens, num_splits, rows, threads)

    def merge(self, partial_o, partial_lse):
        return _merge(self.lib, partial_o, partial_lse)

    def append(self, k_pool, v_pool, page_size, strides, k_new, v_new, block_tables,
               context_lens, query_start_loc=None):
        return _append(self.lib, k_pool, v_pool, page_size, strides, k_new, v_new,
                       block_tables, context_lens, query_start_loc)


def default() -> Oracle:
    global _default
    if _default is None:
        build()
        _default = Oracle(_LIB)
    return _default


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


class PagedInputs:
    """Host copies of one paged-attention problem, as the oracle reads it.

    q: uint16 [T, Hq, D]; k_pool, v_pool: uint16, any 4-d or flat array with
    the given element strides (page, token, head), dim stride 1;
    block_tables: int32 [B, max_blocks]; context_lens: int32 [B];
    query_start_loc: int32 [B+1] or None (decode: sequence s owns token s).
    """

    def __init__(self, q, k_pool, v_pool, block_tables, context_lens, query_start_loc,
                 num_kv_heads: int, page_size: int, strides: Sequence[int],
                 scale: float, causal: bool):
        self.q = np.ascontiguousarray(q, dtype=np.uint16)
        self.k_pool = np.ascontiguousarray(k_pool, dtype=np.uint16)
        self.v_pool = np.ascontiguousarray(v_pool, dtype=np.uint16)
        self.block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
        self.context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
        self.query_start_loc = (None if query_start_loc is None
                                else np.ascontiguousarray(query_start_loc, dtype=np.int32))
        if self.q.ndim != 3:
            raise ValueError("q must be [T, Hq, D]")
        if self.block_tables.ndim != 2:
            raise ValueError("block_tables must be [B, max_blocks]")
        self.num_tokens, self.num_q_heads, self.head_dim = self.q.shape
        self.num_kv_heads = int(num_kv_heads)
        self.page_size = int(page_size)
        self.strides = tuple(int(s) for s in strides)
        self.scale = float(scale)
        self.causal = bool(causal)
        self.num_seqs = int(self.context_lens.shape[0])
        if self.query_start_loc is None and self.num_tokens != self.num_seqs:
            raise ValueError("decode layout needs one query token per sequence")
        if self.query_start_loc is not None and int(self.query_start_loc[-1]) != self.num_tokens:
            raise ValueError("query_start_loc[-1] must equal the number of query tokens")

    def _common(self):
        return [self.num_seqs, self.num_q_heads, self.num_kv_heads, self.head_dim,
                self.page_size, _ptr(self.q), _ptr(self.query_start_loc),
                _ptr(self.k_pool), _ptr(self.v_pool), self.strides[0], self.strides[1],
                self.strides[2], _ptr(self.block_tables), int(self.block_tables.shape[1]),
                _ptr(self.context_lens), self.scale, int(self.causal)]


def _rows_arg(inp: PagedInputs, rows):
    if rows is None:
        return None, inp.num_tokens * inp.num_q_heads
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= inp.num_tokens * inp.num_q_heads):
        raise ValueError("row index out of range")
    return r, int(r.size)


def _attention(lib, inp: PagedInputs, rows=None, threads: Optional[int] = None):
    r, n = _rows_arg(inp, rows)
    out = np.zeros((n, inp.head_dim), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    rc = lib.pa_oracle_attention(*inp._common(), _ptr(r), n, _ptr(out), _ptr(lse),
                                 threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"pa_oracle_attention failed ({rc})")
    return out, lse


def _partials(lib, inp: PagedInputs, split_tokens: int, num_splits: int, rows=None,
              threads: Optional[int] = None):
    r, n = _rows_arg(inp, rows)
    out = np.zeros((n, num_splits, inp.head_dim), dtype=np.float64)
    lse = np.zeros((n, num_splits), dtype=np.float64)
    rc = lib.pa_oracle_partials(*inp._common(), int(split_tokens), int(num_splits), _ptr(r),
                                n, _ptr(out), _ptr(lse), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"pa_oracle_partials failed ({rc})")
    return out, lse


def _merge(lib, partial_o, partial_lse):
    po = np.ascontiguousarray(partial_o, dtype=np.float64)
    pl = np.ascontiguousarray(partial_lse, dtype=np.float64)
    rows, S, D = po.shape
    if pl.shape != (rows, S):
        raise ValueError("partial_lse must be [rows, S]")
    out = np.zeros((rows, D), dtype=np.float64)
    lse = np.zeros((rows,), dtype=np.float64)
    rc = lib.pa_oracle_merge(_ptr(po), _ptr(pl), rows, S, D, _ptr(out), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"pa_oracle_merge failed ({rc})")
    return out, lse


def _append(lib, k_pool, v_pool, page_size, strides, k_new, v_new, block_tables,
            context_lens, query_start_loc=None):
    kp = np.array(k_pool, dtype=np.uint16, copy=True, order="C")
    vp = np.array(v_pool, dtype=np.uint16, copy=True, order="C")
    if kp.shape != vp.shape:
        raise ValueError("K and V pools must have one shape")
    kn = np.ascontiguousarray(k_new, dtype=np.uint16)
    vn = np.ascontiguousarray(v_new, dtype=np.uint16)
    if kn.ndim != 3 or kn.shape != vn.shape:
        raise ValueError("k_new and v_new must be [T, Hkv, D] of one shape")
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qsl = None if query_start_loc is None else np.ascontiguousarray(query_start_loc,
                                                                    dtype=np.int32)
    B = int(cl.shape[0])
    T = B if qsl is None else int(qsl[-1])
    if kn.shape[0] != T:
        raise ValueError("k_new rows must match the new tokens")
    rc = lib.pa_oracle_append(B, int(kn.shape[1]), int(kn.shape[2]), int(page_size),
                              _ptr(kn), _ptr(vn),
                              _ptr(qsl), _ptr(kp), _ptr(vp), int(kp.size), int(strides[0]),
                              int(strides[1]), int(strides[2]), _ptr(bt), int(bt.shape[1]),
                              _ptr(cl))
    if rc != 0:
        raise RuntimeError(f"pa_oracle_append failed ({rc})")
    return kp, vp


def attention(inp: PagedInputs, rows=None, threads: Optional[int] = None):
    """Single-pass attention.  rows: flat indices token*Hq + head, or None for
    every (token, head).  Returns (out fp64 [n, D], lse fp64 [n])."""
    return default().attention(inp, rows, threads)


def partials(inp: PagedInputs, split_tokens: int, num_splits: int, rows=None,
             threads: Optional[int] = None):
    """Split k covers logical tokens [k*split_tokens, (k+1)*split_tokens), cut
    by the allowed set.  Returns (O_k fp64 [n, S, D], lse_k fp64 [n, S])."""
    return default().partials(inp, split_tokens, num_splits, rows, threads)


def merge(partial_o, partial_lse):
    """Log-sum-exp merge of [rows, S, D] partials.  Returns (O [rows, D], LSE [rows])."""
    return default().merge(partial_o, partial_lse)


def append(k_pool, v_pool, page_size, strides, k_new, v_new, block_tables, context_lens,
           query_start_loc=None):
    """Paged KV append on copies of the pools (uint16 bf16 bits, any shape;
    element (page, slot, head, d) at the given (page, token, head) strides,
    d stride 1).  Returns the written copies (k_pool, v_pool)."""
    return default().append(k_pool, v_pool, page_size, strides, k_new, v_new, block_tables,
                            context_lens, query_start_loc)
