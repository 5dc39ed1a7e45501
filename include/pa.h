/*
 * pa.h - C ABI of the MI355X (gfx950) paged grouped-query attention library.
 *
 * Pages cited (by short name):
 *   [IBM-PA]  "一行 Triton 代码同时跑赢 NVIDIA 和 AMD：IBM Research 把大模型推理的
 *             「硬件鸿沟」填平了" (papers.ananclaw.com, summary of arXiv 2511.11581)
 *   [GUIDE]   "从兆字节到兆瓦：基于CUDA与Triton的高性能LLM与扩散内核全指南"
 *             (zhxwu.com GPU programming guide)
 *
 * The operation: for every query token t of sequence s and query head h,
 *   out[t, h, :] = softmax_j( scale * q[t, h, :] . K_s[j, h / G, :] ) V_s[j, h / G, :]
 * over the allowed keys j of that sequence (the SDPA definition, [GUIDE]
 * section "拆解多头注意力（MHA）"), where G = num_q_heads / num_kv_heads groups
 * query heads onto a shared KV head ([IBM-PA] five-step list, Q-Block step),
 * and K_s, V_s are read through the sequence's block table from paged pools
 * ([IBM-PA] model-feature list: paged KV cache, prefix cache).
 * Allowed keys: j < context_lens[s]; with causal set, also
 * j <= context_lens[s] - q_len(s) + i for the i-th new query token of s
 * (future scores are minus infinity, [GUIDE] section "Triton实现Flash
 * Attention", causal item; the new tokens are the last q_len(s) positions of
 * the context, so a chunk attends to the cached prefix and causally to itself).
 * No allowed key: out = 0, lse = -inf.
 *
 * Layouts (element = one bf16 unless stated):
 *   q, out        packed [T, Hq, D], row-major, T query tokens
 *   k_pool/v_pool element (page, slot, kv_head, d) sits at
 *                 page*kv_stride_page + slot*kv_stride_token
 *                 + kv_head*kv_stride_head + d   (d stride is 1)
 *                 K and V share the strides.  Token-major storage is
 *                 [pages, P, Hkv, D]; head-major storage [pages, Hkv, P, D]
 *                 (kv_stride_head = P*D, kv_stride_token = D) keeps a head's
 *                 slots of a page in one run, which the decode kernels
 *                 stream faster on gfx950 (same results, bit for bit).
 *                 Each stride, and P * kv_stride_token, must be below 2^31
 *                 elements, and max_blocks_per_seq * P / 16 below 2^31
 *                 (PA_ERR_UNSUPPORTED otherwise).
 *   block_tables  int32 [B, max_blocks_per_seq]; entry b of row s is the
 *                 page holding logical tokens [b*P, (b+1)*P) of sequence s.
 *                 Entries past ceil(context_lens[s]/P) are never read.
 *   context_lens  int32 [B]; the cached tokens of s, new tokens included.
 *   query_start_loc int32 [B+1] (prefill): tokens of s are rows
 *                 [query_start_loc[s], query_start_loc[s+1]) of q and out.
 *   lse           fp32 [T, Hq], natural log of the softmax denominator
 *                 sum_j exp(scale * q.k_j); optional (NULL to skip).  When it
 *                 is requested, kernels that round the weights P to bf16 for
 *                 the P.V product carry them as bf16 high part + remainder
 *                 instead (variant bit 0 below), so the LSE is not limited by
 *                 bf16's 8-bit significand.
 *
 * Ownership and threading: every pointer is device memory owned by the
 * caller.  The compute calls never allocate, free or synchronise; they only
 * enqueue kernels on the caller's stream, so they can be captured in a HIP
 * graph.  Lengths, tables and query_start_loc are read on the device only;
 * the grid depends only on host fields of pa_problem (a static launch grid,
 * [IBM-PA] five-step list, static-grid and graph steps).  The library's
 * mutable global state is (1) a cache of occupancy figures (compute units
 * x resident workgroups per unit, for the kernels whose grid is sized to
 * the chip), kept per device and keyed on the device of the call's stream,
 * each entry filled on first use with a relaxed atomic store (concurrent
 * first calls compute and store the same value); and (2) for
 * pa_decode_noalloc only, a PA_NOALLOC_SCRATCH_BYTES device array that
 * every GPU holds until the process ends, with its per-device address
 * cached the same way, and whose contents calls on one GPU share (see that
 * entry point).  The tile table is constant.
 *
 * Errors: every host-side argument is checked before anything is enqueued;
 * a failed check returns a status and enqueues nothing.  A failed launch
 * returns PA_ERR_HIP.  Device-side data is trusted: a block-table entry
 * outside the pool, a context longer than max_context_len or than
 * max_blocks_per_seq*P, or a query length above max_query_len is undefined
 * behaviour (pa_check_inputs reports each of these).  Nothing aborts and no
 * exception crosses the ABI.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment          */
  PA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim not 64/128/256,
                             page size < 16, G not in {1,2,4,8,16,32}       */
  PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required     */
  PA_ERR_HIP = 4          /* a HIP launch failed                            */
} pa_status;

typedef enum pa_dtype { PA_BF16 = 0, PA_FP32 = 1 } pa_dtype;

/* Host description of one call.  Every field is read on the host only. */
typedef struct pa_problem {
  int32_t num_seqs;           /* B >= 0                                         */
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads                 */
  int32_t num_kv_heads;       /* Hkv                                            */
  int32_t head_dim;           /* D: 64, 128 or 256 (see PA_ERR_UNSUPPORTED)     */
  int32_t page_size;          /* P, a power of two; 16, 32, 64, ... are built   */
  int32_t max_blocks_per_seq; /* row stride of block_tables                     */
  int64_t kv_stride_page;     /* pool strides in elements, multiples of 8       */
  int64_t kv_stride_token;
  int64_t kv_stride_head;
  int32_t max_context_len;    /* bound on every context_lens[s] (sizes the grid) */
  int32_t max_query_len;      /* bound on every query length; 1 for decode      */
  int32_t total_query_tokens; /* T: rows of q and out                           */
  int32_t causal;             /* 0 or 1 (decode rows are unaffected)            */
  float scale;                /* multiplies q.k, finite and > 0; e.g. 1/sqrt(D)  */
  pa_dtype out_dtype;         /* PA_BF16 or PA_FP32                             */
} pa_problem;

/* Launch shape chosen by pa_select_tiles (or forced by a tuning sweep). */
typedef struct pa_tiles {
  int32_t kv_tile;           /* keys per inner step (16 decode, 32 prefill)      */
  int32_t num_splits;        /* split-KV count S of decode rows (>= 1)           */
  int32_t waves_per_wg;      /* wavefronts per workgroup                         */
  int32_t q_tokens_per_tile; /* query tokens per prefill workgroup               */
  int32_t variant;           /* bit 0 (prefill): carry P as a bf16 high part plus a  */
                             /* bf16 remainder in P.V (relative weight error <=     */
                             /* 2^-16 instead of <= 2^-8); chosen for fp32 outputs, */
                             /* and implied by a non-NULL lse.                       */
                             /* bit 1 (decode, S > 1): merge the splits in a second  */
                             /* kernel instead of in the last workgroup of each      */
                             /* sequence                                             */
                             /* bit 2 (decode, S > 1, needs bit 1): even-work grid: */
                             /* a fixed number of workgroups share all tiles of all */
                             /* sequences equally (cut at any tile, merged by lse);  */
                             /* a sequence is cut into at most S + 1 pieces          */
                             /* bit 3 (one token per sequence, G <= 16): run the     */
                             /* rows on the short-run kernel (pa_prefill's MFMA P.V  */
                             /* path, even-work grid, workspace always needed) in    */
                             /* place of the decode kernels; never the table's       */
                             /* choice: on gfx950 it is within a few per cent of the */
                             /* decode kernels on long batches either way and slower */
                             /* on short ones                                        */
  int32_t tile_splits;       /* pa_prefill: each query tile's keys are cut into     */
                             /* this many runs of whole 32-key tiles (0 or 1: one   */
                             /* run, at most 8), merged by log-sum-exp; it spreads  */
                             /* a few long-prefix chunks over the whole chip, and    */
                             /* the long single-token tiles of mixed batches that   */
                             /* have no decode workgroups                            */
} pa_tiles;

/* Pick the launch shape for a problem from the built-in table (the offline
 * decision table of [IBM-PA] section on moving autotuning offline), and the
 * workspace size the compute call needs.  Pure host code: no HIP call.
 * out and workspace_bytes may not be NULL. */
pa_status pa_select_tiles(const pa_problem* problem, pa_tiles* out, size_t* workspace_bytes);

/* Workspace bytes a given launch shape needs (0 when num_splits == 1). */
pa_status pa_workspace_size(const pa_problem* problem, const pa_tiles* tiles,
                            size_t* workspace_bytes);

/* Decode: one query token per sequence (T = num_seqs, row s of q belongs to
 * sequence s; causal has no effect).  Split-KV ([IBM-PA] five-step list,
 * parallel tiled softmax step): with tiles->num_splits = S > 1 the context of
 * each sequence is cut into S contiguous ranges of whole 16-key tiles
 * processed by different workgroups; their (normalised output, lse) partials go to the
 * workspace and are merged by log-sum-exp in the same call.
 * With tiles->variant bit 1 set (the table's choice) a second kernel merges
 * them: the one behind pa_splitkv_reduce, or on the even-work grid a merge
 * with one workgroup per (sequence, kv head); with it clear the merge runs
 * inside the same launch: the last workgroup of a (sequence, kv head) to
 * finish, found with an atomic arrival counter, merges that sequence's
 * partials, so the call is one kernel.
 * q: bf16 [B, Hq, D]; out: [B, Hq, D] of problem->out_dtype; lse: fp32
 * [B, Hq] or NULL.  workspace: >= pa_workspace_size bytes, 256-byte aligned,
 * may be NULL when that size is 0.  It holds the partials and the arrival
 * counters: it must be zero-filled before its first use, and every call
 * leaves the counters zero again, so it can be reused (and captured) without
 * clearing.  Calls that share one workspace must not run concurrently.
 * tiles->waves_per_wg is 4 or 8.  Pointers to bf16 data must
 * be 16-byte aligned.  problem->max_query_len must be 0 or 1.
 * G = 32 (the decode kernels hold at most 16 query heads per KV head) runs
 * on the short-run kernel described at pa_prefill: one token of 32 heads is
 * a 32-row Q-block, the even-work grid always applies (waves_per_wg and the
 * merge bits are ignored) and the workspace is always needed; so does
 * tiles->variant bit 3 at any G. */
pa_status pa_decode(const pa_problem* problem, const pa_tiles* tiles, const void* q,
                    const void* k_pool, const void* v_pool, const int32_t* block_tables,
                    const int32_t* context_lens, void* out, float* lse, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* Bytes of the scratch array behind pa_decode_noalloc, on each GPU. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* pa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The split partials, piece counts and
 * merge counters that pa_decode keeps in the caller's workspace live here in
 * a file-scope device array of PA_NOALLOC_SCRATCH_BYTES (64 MiB), which the
 * library holds on every GPU it runs on until the process ends.  Arguments,
 * kernels and results are those of pa_decode; the caller still passes the
 * inputs and outputs.
 * Errors: as pa_decode, plus PA_ERR_WORKSPACE (nothing enqueued) when
 * pa_workspace_size for this problem and launch shape exceeds
 * PA_NOALLOC_SCRATCH_BYTES (e.g. 256 sequences at 8k context with the
 * table's 128 splits), and PA_ERR_HIP when the array's device address
 * cannot be found.  Nothing is allocated or freed, by this call or by the
 * library on its behalf.
 * Sharing: every call on one GPU uses that GPU's one array.  Calls that
 * overlap on one GPU (other streams, other threads) race and their results
 * are undefined; calls ordered on one stream are safe.  The array keeps the
 * last call's contents: what a call needs at zero (the arrival counters of
 * the fused merge, variant bit 1 clear) it clears itself with a fill kernel
 * before the decode kernel, and everything else it reads it has written
 * itself.  The first call on a GPU looks the array's address up (with that
 * GPU made current for the lookup, then the caller's device restored):
 * make that first call outside any graph capture. */
pa_status pa_decode_noalloc(const pa_problem* problem, const pa_tiles* tiles, const void* q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens, void* out,
                            float* lse, hipStream_t stream);

/* Prefill / chunked prefill / mixed batch in one launch: sequence s owns
 * query rows [query_start_loc[s], query_start_loc[s+1]); those tokens are
 * the last q_len(s) positions of its context (already written to the pages),
 * so they attend to the cached prefix and, with causal set, causally to each
 * other.  Query length 1 rows (decode sequences) may be mixed in, in any
 * order, as one launch ([IBM-PA], unified kernel for mixed batches):
 * sequences with more than one query token are cut into tiles of
 * q_tokens_per_tile tokens x G heads (a 256-row Q-block, 128 rows at head
 * dim 256), each walking its allowed keys; when the bounds admit
 * single-token sequences (max_query_len <= 1, or total_query_tokens <
 * num_seqs * max_query_len), G <= 8 and head_dim is 128, the same launch
 * also holds split-KV decode workgroups for every (sequence, kv head,
 * split), which return at once for sequences whose query length is not 1.
 * Their partials are merged by a second kernel when tiles->num_splits > 1.
 * Otherwise (G = 16 or 32, head dims 64 and 256) single-token sequences
 * take the tile path, one tile each; pa_select_tiles then splits the query
 * tiles' keys (tile_splits, about 32 * head_dim keys a run) so that the
 * longest such tile does not set the launch time.
 * The host picks the kernels from the problem's bounds alone:
 *   - max_query_len <= 1 (G <= 16): the decode kernels, with query_start_loc
 *     mapping the rows (sequences with no query token are skipped);
 *   - short query runs, 2 <= max_query_len and max_query_len * G <= 64
 *     (speculative-decode verification, [IBM-PA] model-feature list), and
 *     max_query_len <= 1 at G = 32: every (sequence, kv head) unit is one
 *     Q-block of q_len(s) tokens x G heads, streamed over the decode path's
 *     even-work grid (tiles->num_splits bounds the pieces of a unit, S + 1
 *     partial slots per (token, head) row; waves_per_wg, q_tokens_per_tile
 *     and tile_splits are ignored), and a second kernel merges the units cut
 *     into several pieces;
 *   - otherwise the query-tile launch described above.
 * q: bf16 [T, Hq, D]; out: [T, Hq, D] of out_dtype; lse: fp32 [T, Hq] or NULL.
 * With tiles->tile_splits > 1 every query tile's keys are split as well and
 * its partials ([T * Hq, tile_splits, D] fp32 plus lse) are merged by a
 * further kernel.
 * workspace: >= pa_workspace_size bytes (decode-row partials for
 * num_seqs * Hq rows, tile partials for T * Hq rows, or short-run partials
 * for T * Hq rows), zero-filled before first use, as for pa_decode. */
pa_status pa_prefill(const pa_problem* problem, const pa_tiles* tiles, const void* q,
                     const int32_t* query_start_loc, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* context_lens, void* out,
                     float* lse, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Log-sum-exp merge of split partials (the merge that makes the parallel
 * tiled softmax of [IBM-PA] exact; its algebra is that of the online-softmax
 * statistics m and l, [GUIDE] section "Flash Attention革命").  Per row r:
 *   M = max_k lse_k; w_k = exp(lse_k - M);
 *   out[r] = sum_k w_k O_k / sum_k w_k;  lse_out[r] = M + ln sum_k w_k;
 *   every lse_k = -inf gives out[r] = 0 and lse_out[r] = -inf.
 * partial_o: fp32 [rows, S, head_dim] (normalised per split); partial_lse:
 * fp32 [rows, S]; out: [rows, head_dim] of out_dtype; lse_out: fp32 [rows]
 * or NULL.  head_dim must be a positive multiple of 4 (at most 1024),
 * 1 <= num_splits <= 4096; partial_o and out 16-byte aligned. */
pa_status pa_splitkv_reduce(const float* partial_o, const float* partial_lse, int32_t rows,
                            int32_t num_splits, int32_t head_dim, void* out,
                            pa_dtype out_dtype, float* lse_out, hipStream_t stream);

/* Paged KV append: the step just before attention that writes the new
 * tokens' K and V into their block-table slots, so a chunk attends to its
 * prefix and to itself from the pages ([IBM-PA] model-feature list: paged KV
 * cache with prefix caching; the cache layout is that of pa_prefill).
 * Token i of sequence s (0 <= i < q_len(s)) goes to logical position
 * p = context_lens[s] - q_len(s) + i, i.e. page block_tables[s][p / P],
 * slot p % P, kv head h, at page*kv_stride_page + slot*kv_stride_token +
 * h*kv_stride_head; context_lens counts the new tokens, as for pa_prefill.
 * k_new, v_new: bf16 [T, Hkv, D] (row t = one token, D contiguous), rows in
 * query_start_loc order; query_start_loc NULL means one token per sequence
 * (T = num_seqs, decode).  T = problem->total_query_tokens.  k_pool,
 * v_pool: the caller's paged pools, written only at those slots.  Every
 * block-table entry a token lands in must be a valid page of the pools; a
 * sequence with context_lens[s] < q_len(s) is undefined.  Rows past their
 * sequence's tokens, positions past the table row and negative table entries
 * write nothing.
 * Pointers to bf16 data must be 16-byte aligned.  Host checks as for the
 * other calls; nothing is allocated. */
pa_status pa_cache_append(const pa_problem* problem, const void* k_new, const void* v_new,
                          const int32_t* query_start_loc, const int32_t* block_tables,
                          const int32_t* context_lens, void* k_pool, void* v_pool,
                          hipStream_t stream);

/* Bits pa_check_inputs reports. */
typedef enum {
  PA_CHECK_PAGE = 1,           /* a block-table entry a context uses is outside [0, num_pages) */
  PA_CHECK_CONTEXT_BOUND = 2,  /* context_lens[s] < 0 or > max_context_len                     */
  PA_CHECK_CONTEXT_BLOCKS = 4, /* context_lens[s] > max_blocks_per_seq * page_size              */
  PA_CHECK_QUERY_STARTS = 8,   /* query_start_loc not rising from 0 to total_query_tokens      */
  PA_CHECK_QUERY_LEN = 16,     /* a query length above max_query_len                            */
  PA_CHECK_CONTEXT_SHORT = 32  /* a sequence with more query tokens than context: its new
                                  tokens have no positions.  Undefined for pa_cache_append
                                  (which writes nothing for them); defined for attention, whose
                                  rows before position 0 see no key (O = 0, lse = -inf), as a
                                  decode row of an empty context does                          */
} pa_check_flag;

/* The compute calls trust the device-side tables and lengths: they only
 * clamp, so that bad values cannot take them outside the block table or the
 * workspace, and the results are then undefined.  This call checks them
 * instead, for the problem a pa_decode, pa_prefill or pa_cache_append call
 * would be given (the paged cache of the [IBM-PA] model-feature list:
 * page = block_tables[s][t / P] for every token t < context_lens[s]).
 * Enqueued on stream: *flags (device int32) is cleared, then gets the OR of
 * the PA_CHECK_* bits of every failed check; the caller reads it after
 * synchronising.  num_pages: pages in the K/V pools.  query_start_loc: as for
 * pa_prefill, or NULL for one token per sequence.  block_tables and
 * context_lens as for the compute calls.  Host arguments are checked first
 * (PA_ERR_INVALID_ARG, nothing enqueued); nothing is allocated. */
pa_status pa_check_inputs(const pa_problem* problem, int64_t num_pages,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start_loc, int32_t* flags, hipStream_t stream);

/* Static text for a status code. */
const char* pa_status_string(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
