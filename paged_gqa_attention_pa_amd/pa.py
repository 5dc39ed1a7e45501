"""Thin Python binding of libpa.so (include/pa.h): argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI;
PyTorch only provides device memory and the current stream.  If libpa.so is
missing or cannot be loaded, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
_lib = None

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(5)
PA_BF16, PA_FP32 = 0, 1

EXPORTED = ["pa_select_tiles", "pa_workspace_size", "pa_decode", "pa_decode_noalloc",
            "pa_prefill", "pa_splitkv_reduce", "pa_cache_append", "pa_check_inputs",
            "pa_status_string"]
NOALLOC_SCRATCH_BYTES = 64 << 20  # PA_NOALLOC_SCRATCH_BYTES
# pa_check_inputs bits
CHECK_PAGE, CHECK_CONTEXT_BOUND, CHECK_CONTEXT_BLOCKS = 1, 2, 4
CHECK_QUERY_STARTS, CHECK_QUERY_LEN, CHECK_CONTEXT_SHORT = 8, 16, 32


class Problem(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("kv_stride_page", ctypes.c_int64), ("kv_stride_token", ctypes.c_int64),
                ("kv_stride_head", ctypes.c_int64), ("max_context_len", ctypes.c_int32),
                ("max_query_len", ctypes.c_int32), ("total_query_tokens", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("out_dtype", ctypes.c_int32)]


class Tiles(ctypes.Structure):
    _fields_ = [("kv_tile", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("waves_per_wg", ctypes.c_int32), ("q_tokens_per_tile", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("tile_splits", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libpa.so; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run "
                              "`python -m paged_gqa_attention_pa_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, PP = ctypes.c_void_p, ctypes.POINTER
        lib.pa_select_tiles.argtypes = [PP(Problem), PP(Tiles), PP(ctypes.c_size_t)]
        lib.pa_workspace_size.argtypes = [PP(Problem), PP(Tiles), PP(ctypes.c_size_t)]
        lib.pa_decode.argtypes = [PP(Problem), PP(Tiles), P, P, P, P, P, P, P, P,
                                  ctypes.c_size_t, P]
        lib.pa_decode_noalloc.argtypes = [PP(Problem), PP(Tiles), P, P, P, P, P, P, P, P]
        lib.pa_prefill.argtypes = [PP(Problem), PP(Tiles), P, P, P, P, P, P, P, P, P,
                                   ctypes.c_size_t, P]
        lib.pa_splitkv_reduce.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          P, ctypes.c_int32, P, P]
        lib.pa_cache_append.argtypes = [PP(Problem), P, P, P, P, P, P, P, P]
        lib.pa_check_inputs.argtypes = [PP(Problem), ctypes.c_int64, P, P, P, P, P]
        for f in EXPORTED[:-1]:
            getattr(lib, f).restype = ctypes.c_int
        lib.pa_status_string.argtypes = [ctypes.c_int]
        lib.pa_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().pa_status_string(status).decode()


def _check(status: int, where: str):
    if status != PA_OK:
        raise PAError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_problem(q: torch.Tensor, k_pool: torch.Tensor, block_tables: torch.Tensor,
                 num_seqs: int, scale: float, max_context_len: int, max_query_len: int,
                 causal: bool = True, out_dtype: torch.dtype = torch.bfloat16) -> Problem:
    """pa_problem for packed q [T, Hq, D] and a pool laid out (page, slot,
    kv_head, dim) with any strides (dim stride 1)."""
    if q.dim() != 3 or k_pool.dim() != 4:
        raise ValueError("q must be [T, Hq, D] and the pools [pages, P, Hkv, D]")
    if k_pool.stride(3) != 1:
        raise ValueError("pool dim stride must be 1")
    T, Hq, D = q.shape
    _, P, Hkv, D2 = k_pool.shape
    if D2 != D:
        raise ValueError("head_dim of q and the pools differ")
    pb = Problem()
    pb.num_seqs = int(num_seqs)
    pb.num_q_heads, pb.num_kv_heads, pb.head_dim, pb.page_size = int(Hq), int(Hkv), int(D), int(P)
    pb.max_blocks_per_seq = int(block_tables.shape[1])
    pb.kv_stride_page, pb.kv_stride_token, pb.kv_stride_head = (int(k_pool.stride(0)),
                                                              int(k_pool.stride(1)),
                                                              int(k_pool.stride(2)))
    pb.max_context_len = int(max_context_len)
    pb.max_query_len = int(max_query_len)
    pb.total_query_tokens = int(T)
    pb.causal = int(bool(causal))
    pb.scale = float(scale)
    if out_dtype == torch.bfloat16:
        pb.out_dtype = PA_BF16
    elif out_dtype == torch.float32:
        pb.out_dtype = PA_FP32
    else:
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    return pb


def select_tiles(problem: Problem) -> Tuple[Tiles, int]:
    t = Tiles()
    ws = ctypes.c_size_t(0)
    _check(load().pa_select_tiles(ctypes.byref(problem), ctypes.byref(t), ctypes.byref(ws)),
           "pa_select_tiles")
    return t, int(ws.value)


def workspace_size(problem: Problem, tiles: Tiles) -> int:
    ws = ctypes.c_size_t(0)
    _check(load().pa_workspace_size(ctypes.byref(problem), ctypes.byref(tiles), ctypes.byref(ws)),
           "pa_workspace_size")
    return int(ws.value)


def _check_tensors(q, k_pool, v_pool, block_tables, context_lens, out, lse):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    for name, t, dt in [("q", q, torch.bfloat16), ("k_pool", k_pool, torch.bfloat16),
                        ("v_pool", v_pool, torch.bfloat16),
                        ("block_tables", block_tables, torch.int32),
                        ("context_lens", context_lens, torch.int32)]:
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt}")
    if not q.is_contiguous() or not block_tables.is_contiguous() or not context_lens.is_contiguous():
        raise ValueError("q, block_tables and context_lens must be contiguous")
    if k_pool.shape != v_pool.shape or k_pool.stride() != v_pool.stride():
        raise ValueError("K and V pools must share shape and strides")
    if out.device != dev or not out.is_contiguous() or out.shape != q.shape:
        raise ValueError("out must be a contiguous tensor shaped like q on q's device")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.device != dev or tuple(lse.shape) != tuple(q.shape[:2])):
        raise ValueError("lse must be contiguous fp32 [T, Hq] on q's device")


def _check_problem(problem: Problem, q: torch.Tensor, out: torch.Tensor, k_pool: torch.Tensor,
                   block_tables: torch.Tensor, num_seqs: int):
    """A caller-built pa_problem must describe the tensors actually passed."""
    odt = PA_FP32 if out.dtype == torch.float32 else PA_BF16
    if problem.out_dtype != odt:
        raise ValueError("problem.out_dtype does not match out.dtype")
    T, Hq, D = q.shape
    if (problem.total_query_tokens != T or problem.num_q_heads != Hq or problem.head_dim != D
            or problem.num_seqs != num_seqs or problem.num_kv_heads != k_pool.shape[2]
            or problem.page_size != k_pool.shape[1]
            or problem.max_blocks_per_seq != block_tables.shape[1]
            or (problem.kv_stride_page, problem.kv_stride_token, problem.kv_stride_head)
            != tuple(int(x) for x in k_pool.stride()[:3])):
        raise ValueError("problem does not match the tensors' shapes or strides")


def decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
           max_context_len: int, out: Optional[torch.Tensor] = None,
           out_dtype: torch.dtype = torch.bfloat16, lse: Optional[torch.Tensor] = None,
           tiles: Optional[Tiles] = None, workspace: Optional[torch.Tensor] = None,
           problem: Optional[Problem] = None) -> torch.Tensor:
    """pa_decode: q [B, Hq, D] bf16 (one query token per sequence).

    A caller-provided workspace must have been zero-filled once (its split
    counters); every call leaves it reusable."""
    lib = load()
    B = q.shape[0]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _check_tensors(q, k_pool, v_pool, block_tables, context_lens, out, lse)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("decode needs one block-table row and one length per query row")
    if problem is None:
        problem = make_problem(q, k_pool, block_tables, B, scale, max_context_len, 1,
                               causal=True, out_dtype=out.dtype)
    else:
        _check_problem(problem, q, out, k_pool, block_tables, B)
    if tiles is None:
        tiles, ws = select_tiles(problem)
    else:
        ws = workspace_size(problem, tiles)
    if ws and workspace is None:
        workspace = torch.zeros(ws, dtype=torch.uint8, device=q.device)  # counters start at 0
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pa_decode(ctypes.byref(problem), ctypes.byref(tiles), _ptr(q), _ptr(k_pool),
                         _ptr(v_pool), _ptr(block_tables), _ptr(context_lens), _ptr(out),
                         _ptr(lse), _ptr(workspace), wsb, _stream(q.device)), "pa_decode")
    return out


def decode_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                   max_context_len: int, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                   tiles: Optional[Tiles] = None,
                   problem: Optional[Problem] = None) -> torch.Tensor:
    """pa_decode_noalloc: pa_decode with the library's per-GPU scratch array
    in place of a workspace.  `out` must be given (this call allocates no
    device memory; tiles come from pa_select_tiles when None, a host-only
    lookup)."""
    lib = load()
    B = q.shape[0]
    _check_tensors(q, k_pool, v_pool, block_tables, context_lens, out, lse)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("decode needs one block-table row and one length per query row")
    if problem is None:
        problem = make_problem(q, k_pool, block_tables, B, scale, max_context_len, 1,
                               causal=True, out_dtype=out.dtype)
    else:
        _check_problem(problem, q, out, k_pool, block_tables, B)
    if tiles is None:
        tiles, _ = select_tiles(problem)
    _check(lib.pa_decode_noalloc(ctypes.byref(problem), ctypes.byref(tiles), _ptr(q),
                                 _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                 _ptr(context_lens), _ptr(out), _ptr(lse), _stream(q.device)),
           "pa_decode_noalloc")
    return out


def prefill(q: torch.Tensor, query_start_loc: torch.Tensor, k_pool: torch.Tensor,
            v_pool: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
            scale: float, max_context_len: int, max_query_len: int, causal: bool = True,
            out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
            lse: Optional[torch.Tensor] = None, tiles: Optional[Tiles] = None,
            workspace: Optional[torch.Tensor] = None,
            problem: Optional[Problem] = None) -> torch.Tensor:
    """pa_prefill: q [T, Hq, D] bf16; sequence s owns rows
    [query_start_loc[s], query_start_loc[s+1])."""
    lib = load()
    B = context_lens.shape[0]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _check_tensors(q, k_pool, v_pool, block_tables, context_lens, out, lse)
    if (query_start_loc.dtype != torch.int32 or query_start_loc.device != q.device
            or query_start_loc.shape[0] != B + 1 or not query_start_loc.is_contiguous()):
        raise ValueError("query_start_loc must be contiguous int32 [B+1] on q's device")
    if block_tables.shape[0] != B:
        raise ValueError("block_tables needs one row per sequence")
    if problem is None:
        problem = make_problem(q, k_pool, block_tables, B, scale, max_context_len,
                               max_query_len, causal=causal, out_dtype=out.dtype)
    else:
        _check_problem(problem, q, out, k_pool, block_tables, B)
    if tiles is None:
        tiles, ws = select_tiles(problem)
    else:
        ws = workspace_size(problem, tiles)
    if ws and workspace is None:
        workspace = torch.zeros(ws, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pa_prefill(ctypes.byref(problem), ctypes.byref(tiles), _ptr(q),
                          _ptr(query_start_loc), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                          _ptr(context_lens), _ptr(out), _ptr(lse), _ptr(workspace), wsb,
                          _stream(q.device)), "pa_prefill")
    return out


def splitkv_reduce(partial_o: torch.Tensor, partial_lse: torch.Tensor,
                   out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32,
                   lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pa_splitkv_reduce: partial_o fp32 [rows, S, D], partial_lse fp32 [rows, S]."""
    lib = load()
    rows, S, D = partial_o.shape
    if partial_o.dtype != torch.float32 or partial_lse.dtype != torch.float32:
        raise ValueError("partials must be fp32")
    if not partial_o.is_contiguous() or not partial_lse.is_contiguous():
        raise ValueError("partials must be contiguous")
    if tuple(partial_lse.shape) != (rows, S):
        raise ValueError("partial_lse must be [rows, S]")
    if out is None:
        out = torch.empty((rows, D), dtype=out_dtype, device=partial_o.device)
    if out.dtype == torch.float32:
        odt = PA_FP32
    elif out.dtype == torch.bfloat16:
        odt = PA_BF16
    else:
        raise ValueError("out must be fp32 or bf16")
    if tuple(out.shape) != (rows, D) or not out.is_contiguous():
        raise ValueError("out must be contiguous [rows, D]")
    if lse is not None and (tuple(lse.shape) != (rows,) or lse.dtype != torch.float32):
        raise ValueError("lse must be fp32 [rows]")
    _check(lib.pa_splitkv_reduce(_ptr(partial_o), _ptr(partial_lse), rows, S, D, _ptr(out),
                                 odt, _ptr(lse), _stream(partial_o.device)),
           "pa_splitkv_reduce")
    return out


def cache_append(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
                 v_pool: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                 query_start_loc: Optional[torch.Tensor] = None,
                 problem: Optional[Problem] = None) -> None:
    """pa_cache_append: k_new, v_new bf16 [T, Hkv, D]; writes them into the
    pools at the newest q_len(s) positions of each sequence's context
    (query_start_loc None: one token per sequence)."""
    lib = load()
    dev = k_new.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    for name, t, dt in [("k_new", k_new, torch.bfloat16), ("v_new", v_new, torch.bfloat16),
                        ("k_pool", k_pool, torch.bfloat16), ("v_pool", v_pool, torch.bfloat16),
                        ("block_tables", block_tables, torch.int32),
                        ("context_lens", context_lens, torch.int32)]:
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, k_new on {dev}")
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt}")
    if (k_new.dim() != 3 or k_new.shape != v_new.shape or not k_new.is_contiguous()
            or not v_new.is_contiguous()):
        raise ValueError("k_new and v_new must be contiguous [T, Hkv, D] of one shape")
    if k_pool.shape != v_pool.shape or k_pool.stride() != v_pool.stride():
        raise ValueError("K and V pools must share shape and strides")
    if k_pool.dim() != 4 or tuple(k_new.shape[1:]) != tuple(k_pool.shape[2:]):
        raise ValueError("pools must be [pages, P, Hkv, D] with k_new's Hkv and D")
    if not block_tables.is_contiguous() or not context_lens.is_contiguous():
        raise ValueError("block_tables and context_lens must be contiguous")
    B = context_lens.shape[0]
    if block_tables.shape[0] != B:
        raise ValueError("block_tables needs one row per sequence")
    T = k_new.shape[0]
    if query_start_loc is None:
        if T != B:
            raise ValueError("without query_start_loc there is one token per sequence")
    elif (query_start_loc.dtype != torch.int32 or query_start_loc.device != dev
          or query_start_loc.shape[0] != B + 1 or not query_start_loc.is_contiguous()):
        raise ValueError("query_start_loc must be contiguous int32 [B+1] on k_new's device")
    if problem is None:
        problem = make_problem(k_new, k_pool, block_tables, B, 1.0, 0, 1)
    elif (problem.total_query_tokens != T or problem.num_seqs != B
          or problem.num_kv_heads != k_pool.shape[2] or problem.head_dim != k_pool.shape[3]
          or problem.page_size != k_pool.shape[1]
          or problem.max_blocks_per_seq != block_tables.shape[1]
          or (problem.kv_stride_page, problem.kv_stride_token, problem.kv_stride_head)
          != tuple(int(x) for x in k_pool.stride()[:3])):
        raise ValueError("problem does not match the tensors' shapes or strides")
    _check(lib.pa_cache_append(ctypes.byref(problem), _ptr(k_new), _ptr(v_new),
                               _ptr(query_start_loc), _ptr(block_tables), _ptr(context_lens),
                               _ptr(k_pool), _ptr(v_pool), _stream(dev)), "pa_cache_append")


def check_inputs(problem: Problem, num_pages: int, block_tables: torch.Tensor,
                 context_lens: torch.Tensor,
                 query_start_loc: Optional[torch.Tensor] = None) -> int:
    """pa_check_inputs: the OR of the CHECK_* bits of every device-side check
    that fails for this problem (0: tables and lengths are consistent).
    Synchronises the current stream to read the result."""
    lib = load()
    dev = context_lens.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    for name, t in [("block_tables", block_tables), ("context_lens", context_lens),
                    ("query_start_loc", query_start_loc)]:
        if t is None:
            continue
        if t.device != dev or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous int32 on {dev}")
    if block_tables.shape[0] != problem.num_seqs or context_lens.numel() != problem.num_seqs:
        raise ValueError("block_tables and context_lens need one row per sequence")
    if block_tables.shape[1] != problem.max_blocks_per_seq:
        raise ValueError("block_tables row length must be max_blocks_per_seq")
    if query_start_loc is not None and query_start_loc.numel() != problem.num_seqs + 1:
        raise ValueError("query_start_loc needs num_seqs + 1 entries")
    flags = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.pa_check_inputs(ctypes.byref(problem), int(num_pages), _ptr(block_tables),
                               _ptr(context_lens), _ptr(query_start_loc), _ptr(flags),
                               _stream(dev)), "pa_check_inputs")
    return int(flags.item())
