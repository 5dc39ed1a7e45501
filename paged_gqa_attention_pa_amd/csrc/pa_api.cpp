// C ABI of the paged GQA attention library: argument checks, launch-shape
// selection, workspace sizing, and the launches.  Host code only; every
// check runs before anything is enqueued.
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "../../include/pa.h"
#include "pa_internal.h"
#include "pa_tile_table.h"

namespace {

using pa::kHeadDim;
using pa::kPage;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

bool group_built(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32; }

// The 32 bits a caller put in a pa_dtype field or argument.  In C++ reading
// an enum object whose value is none of its enumerators is undefined, so the
// value is copied out as an integer before it is checked.
int32_t raw_dtype(const pa_dtype& d) {
  static_assert(sizeof(pa_dtype) == sizeof(int32_t), "pa_dtype is a 32-bit C enum");
  int32_t v;
  memcpy(&v, &d, sizeof v);
  return v;
}
bool dtype_valid(const pa_dtype& d) {
  const int32_t v = raw_dtype(d);
  return v == PA_BF16 || v == PA_FP32;
}

// Checks shared by every call; returns PA_OK or the first failure.
pa_status check_problem(const pa_problem* pb) {
  if (!pb) return PA_ERR_INVALID_ARG;
  if (pb->num_seqs < 0 || pb->num_q_heads <= 0 || pb->num_kv_heads <= 0 || pb->head_dim <= 0 ||
      pb->page_size <= 0 || pb->max_blocks_per_seq <= 0 || pb->max_context_len < 0 ||
      pb->max_query_len < 0 || pb->total_query_tokens < 0)
    return PA_ERR_INVALID_ARG;
  if (pb->num_q_heads % pb->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if ((pb->page_size & (pb->page_size - 1)) != 0) return PA_ERR_INVALID_ARG;
  if (pb->kv_stride_page <= 0 || pb->kv_stride_token <= 0 || pb->kv_stride_head <= 0 ||
      pb->kv_stride_page % 8 || pb->kv_stride_token % 8 || pb->kv_stride_head % 8)
    return PA_ERR_INVALID_ARG;
  if (!dtype_valid(pb->out_dtype)) return PA_ERR_INVALID_ARG;
  if (pb->causal != 0 && pb->causal != 1) return PA_ERR_INVALID_ARG;
  if (!(pb->scale > 0.f) || pb->scale == __builtin_inff()) return PA_ERR_INVALID_ARG;
  if ((int64_t)pb->max_context_len > (int64_t)pb->max_blocks_per_seq * pb->page_size)
    return PA_ERR_INVALID_ARG;
  if ((pb->head_dim != 64 && pb->head_dim != kHeadDim && pb->head_dim != 256) ||
      pb->page_size < kPage)
    return PA_ERR_UNSUPPORTED;
  // the kernels form page offsets as 32-bit byte strides times page ids, the
  // slot offsets inside a page in 32 bits, and 16-key tile indices (up to
  // max_blocks_per_seq * page_size / 16) as int
  if (pb->kv_stride_page > 0x7fffffff || pb->kv_stride_token > 0x7fffffff ||
      pb->kv_stride_head > 0x7fffffff ||
      (int64_t)pb->kv_stride_token * pb->page_size > 0x7fffffff ||
      (int64_t)pb->max_blocks_per_seq * (pb->page_size / kPage) > 0x7fffffff)
    return PA_ERR_UNSUPPORTED;
  if (!group_built(pb->num_q_heads / pb->num_kv_heads)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// log2 of the page size, and of the 16-key tiles per page (page sizes are
// powers of two from 16, checked above)
int log2_page(const pa_problem* pb) { return __builtin_ctz((unsigned)pb->page_size); }
int page_shift(const pa_problem* pb) { return log2_page(pb) - __builtin_ctz((unsigned)kPage); }

pa_status check_tiles(const pa_tiles* t) {
  if (!t) return PA_ERR_INVALID_ARG;
  if (t->num_splits < 1 || t->num_splits > pa::kMaxSplits) return PA_ERR_INVALID_ARG;
  if (t->tile_splits < 0 || t->tile_splits > pa::kMaxTileSplits) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int tile_splits_of(const pa_problem* pb, const pa_tiles* t) {
  return (pb->max_query_len > 1 && t->tile_splits > 1) ? t->tile_splits : 1;
}

// Workspace, 256-byte aligned regions:
//  decode rows (num_splits > 1): partial O [B*Hq, slots, D] fp32, partial
//    lse [B*Hq, slots] fp32 (slots = S, or S + 1 for the even-work grid), one
//    int32 arrival counter per (sequence, kv head) and one int32 piece count
//    per (sequence, kv head); the arrival counters must be zero before the
//    first call, every call leaves them zero;
//  query tiles (prefill problems, tile_splits > 1): partial O
//    [T*Hq, tile_splits, D] fp32 and partial lse [T*Hq, tile_splits].
// dec_total is the end of the decode-row part (all pa_decode needs).
struct Workspace {
  size_t o_off, lse_off, ctr_off, cnt_off, dec_total, to_off, tlse_off, total;
};

// Short query runs (speculative-decode verification): every sequence of the
// batch has at most max_query_len >= 2 tokens and max_query_len * G <= 64,
// so a (sequence, kv head) unit is one Q-block of at most 64 rows.  Decode
// at G = 32 (32 query heads on one KV head) runs the same way, the decode
// kernels holding at most 16 heads per KV head, and so does decode at head
// dims other than 128.
bool verify_path(const pa_problem* pb) {
  const int G = pb->num_q_heads / pb->num_kv_heads;
  if ((G == 32 || pb->head_dim != kHeadDim) && pb->max_query_len <= 1)
    return pa::verify_row_blocks(G, 1, pb->head_dim) > 0;
  return pb->max_query_len >= 2 && pa::verify_row_blocks(G, pb->max_query_len, pb->head_dim) > 0;
}

pa_status check_attention(const pa_problem* pb) { return check_problem(pb); }

// Query tokens of one query tile: the Q-block (256 rows, 128 at head dim
// 256) over the G heads of a KV head.
int query_tile_tokens(const pa_problem* pb) {
  const int G = pb->num_q_heads / pb->num_kv_heads;
  return (pb->head_dim == 256 ? 128 : 256) / G;
}

// Rows of the short-run partials: (token, q head) pairs; a decode-layout
// problem has one token per sequence.
int64_t short_run_rows(const pa_problem* pb) {
  const int64_t tokens = pb->max_query_len <= 1 ? pb->num_seqs : pb->total_query_tokens;
  return tokens * pb->num_q_heads;
}

// The short-run kernel serves this call: short query runs, decode at G = 32
// or head dims other than 128, and decode batches whose launch shape asks
// for it (variant bit 3).
bool short_path(const pa_problem* pb, const pa_tiles* t) {
  if (verify_path(pb)) return true;
  const int G = pb->num_q_heads / pb->num_kv_heads;
  return pb->max_query_len <= 1 && t && (t->variant & pa::kVariantShortDecode) != 0 &&
         pa::verify_row_blocks(G, 1, pb->head_dim) > 0;
}

bool even_grid(const pa_tiles* t) {
  return t->num_splits > 1 && (t->variant & pa::kVariantEvenWork) != 0;
}

Workspace workspace_layout(const pa_problem* pb, const pa_tiles* t) {
  Workspace w{0, 0, 0, 0, 0, 0, 0, 0};
  const int64_t D = pb->head_dim;
  const int S = t->num_splits;
  const bool verify = short_path(pb, t);
  if (S > 1 || verify) {
    // short query runs: (token, head) rows, always the even-work grid
    const int64_t rows = verify ? short_run_rows(pb) : (int64_t)pb->num_seqs * pb->num_q_heads;
    const int64_t slots = S + ((verify || even_grid(t)) ? 1 : 0);
    const size_t units = (size_t)((int64_t)pb->num_seqs * pb->num_kv_heads);
    w.lse_off = align_up((size_t)(rows * slots * D) * sizeof(float));
    w.ctr_off = w.lse_off + align_up((size_t)(rows * slots) * sizeof(float));
    w.cnt_off = w.ctr_off + align_up(units * sizeof(int32_t));
    w.dec_total = w.cnt_off + align_up(units * sizeof(int32_t));
  }
  const int ts = verify ? 1 : tile_splits_of(pb, t);
  w.total = w.dec_total;
  if (ts > 1) {
    const int64_t rows = (int64_t)pb->total_query_tokens * pb->num_q_heads;
    w.to_off = w.dec_total;
    w.tlse_off = w.to_off + align_up((size_t)(rows * ts * D) * sizeof(float));
    w.total = w.tlse_off + align_up((size_t)(rows * ts) * sizeof(float));
  }
  return w;
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Can a prefill-type batch hold single-token (decode) sequences?  Host
// bounds only: yes unless every sequence has exactly max_query_len tokens.
bool may_hold_decode_rows(const pa_problem* pb) {
  return pb->max_query_len <= 1 ||
         (int64_t)pb->total_query_tokens < (int64_t)pb->num_seqs * pb->max_query_len;
}

// In a unified launch, do the single-token sequences run as split decode
// workgroups beside the query tiles?  Only at head dim 128 and G <= 8 (the
// decode body's shapes); elsewhere each one is a query tile of its own.
bool decode_rows_apart(const pa_problem* pb) {
  const int G = pb->num_q_heads / pb->num_kv_heads;
  return may_hold_decode_rows(pb) && G <= 8 && pb->head_dim == kHeadDim;
}

// Key-run splits of the query tiles of a batch whose single-token sequences
// run as query tiles.  Such a tile holds one token yet walks the whole
// context at the cost of a full tile, so the longest one sets the launch
// time unless its keys are split.  Measured on gfx950 (16 single-token
// sequences with contexts up to 16k beside two 512-token chunks): the best
// runs hold about 32 * head_dim keys (D = 64: 8 splits, 370 -> 245 us;
// G = 16 at D = 128: 4 splits, 536 -> 336 us; D = 256: 2 splits,
// 802 -> 560 us), and splitting further than about eight workgroups per CU
// (2048 in all) only adds partial traffic; that cap gives the D = 64 batch
// 7 splits (249 us).
int mixed_tile_splits(const pa_problem* pb) {
  const int qt = query_tile_tokens(pb);
  const int64_t tiles = ((int64_t)pb->total_query_tokens + qt - 1) / qt + pb->num_seqs;
  const int64_t wgs = tiles * pb->num_kv_heads;
  const int64_t run_keys = 32 * (int64_t)pb->head_dim;
  int64_t s = ((int64_t)pb->max_context_len + run_keys - 1) / run_keys;
  const int64_t s_wgs = 2048 / (wgs > 0 ? wgs : 1);
  if (s > s_wgs) s = s_wgs;
  if (s > pa::kMaxTileSplits) s = pa::kMaxTileSplits;
  return s < 1 ? 1 : (int)s;
}

// pa_prefill for short query runs, and pa_decode at G = 32
// (query_start_loc null): the even-work grid over every (sequence, kv head)
// unit with one Q-block per unit, then the merge of the units cut into
// several pieces.  Arguments were checked by the caller.
pa_status short_runs(const pa_problem* problem, const pa_tiles* tiles, const void* q,
                             const int32_t* query_start_loc, const void* k_pool,
                             const void* v_pool, const int32_t* block_tables,
                             const int32_t* context_lens, void* out, float* lse, char* ws,
                             const Workspace& wl, hipStream_t stream) {
  const int G = problem->num_q_heads / problem->num_kv_heads;
  const int S = tiles->num_splits;
  const int rb = pa::verify_row_blocks(G, problem->max_query_len > 1 ? problem->max_query_len : 1,
                                       problem->head_dim);
  // an LSE is asked for: weights as bf16 high part + remainder, so its
  // denominator is not rounded to bf16's 8-bit significand
  const bool precise = (tiles->variant & pa::kVariantPreciseP) != 0 || lse != nullptr;
  pa::DecodeParams d;
  d.q = static_cast<const uint16_t*>(q);
  d.k_pool = static_cast<const uint16_t*>(k_pool);
  d.v_pool = static_cast<const uint16_t*>(v_pool);
  d.block_tables = block_tables;
  d.context_lens = context_lens;
  d.out = out;
  d.lse = lse;
  d.part_o = reinterpret_cast<float*>(ws + wl.o_off);
  d.part_lse = reinterpret_cast<float*>(ws + wl.lse_off);
  d.counters = reinterpret_cast<int32_t*>(ws + wl.ctr_off);
  d.piece_counts = reinterpret_cast<int32_t*>(ws + wl.cnt_off);
  d.query_start_loc = query_start_loc;
  d.stride_page = problem->kv_stride_page;
  d.stride_token = problem->kv_stride_token;
  d.stride_head = problem->kv_stride_head;
  d.num_seqs = problem->num_seqs;
  d.num_q_heads = problem->num_q_heads;
  d.num_kv_heads = problem->num_kv_heads;
  d.max_blocks = problem->max_blocks_per_seq;
  d.page_shift = page_shift(problem);
  d.num_splits = S + 1;
  const int ntiles = ceil_div(problem->max_context_len, pa::kDecodeTile);
  d.tiles_per_split = ntiles > 0 ? ceil_div(ntiles, S) : 1;
  d.max_tiles = ntiles;
  d.even_min_tiles = d.tiles_per_split;
  d.scale_log2 = problem->scale * pa::kLog2eHost;
  d.out_f32 = problem->out_dtype == PA_FP32;
  d.causal = problem->causal;
  const int nw = pa::verify_resident(G, rb, precise, problem->head_dim, stream);
  if (nw <= 0) return PA_ERR_HIP;
  pa_status st = from_hip(pa::launch_verify(d, G, rb, precise, problem->head_dim, nw, stream));
  if (st != PA_OK) return st;
  pa::ReduceParams r;
  r.part_o = d.part_o;
  r.part_lse = d.part_lse;
  r.out = out;
  r.lse = lse;
  r.rows = problem->total_query_tokens * problem->num_q_heads;
  r.num_splits = d.num_splits;
  r.head_dim = problem->head_dim;
  r.out_f32 = d.out_f32;
  r.query_start_loc = query_start_loc;
  r.num_q_heads = problem->num_q_heads;
  r.piece_counts = d.piece_counts;
  r.context_lens = context_lens;
  r.group = G;
  r.unit_rows = 0;
  const int unit_rows = (problem->max_query_len > 1 ? problem->max_query_len : 1) * G;
  return from_hip(
      pa::launch_unit_merge(r, problem->num_seqs * problem->num_kv_heads, unit_rows, stream));
}

pa_status check_decode(const pa_problem* problem, const pa_tiles* tiles, const void* q,
                       const void* k_pool, const void* v_pool, const int32_t* block_tables,
                       const int32_t* context_lens, const void* out) {
  pa_status st = check_attention(problem);
  if (st != PA_OK) return st;
  if ((st = check_tiles(tiles)) != PA_OK) return st;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PA_ERR_INVALID_ARG;
  if (problem->max_query_len > 1) return PA_ERR_INVALID_ARG;  // one token per sequence
  const int G = problem->num_q_heads / problem->num_kv_heads;
  const int waves = tiles->waves_per_wg;
  if (short_path(problem, tiles)) return PA_OK;  // the short-run kernel ignores the waves
  if (waves != 4 && waves != 8) return PA_ERR_INVALID_ARG;
  // the even-work grid merges in the separate kernel only
  if (even_grid(tiles) && (tiles->variant & pa::kVariantSeparateMerge) == 0)
    return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// Decode on the decode kernels with the fused last-workgroup merge: the
// workspace's arrival counters must be zero when the call starts.
bool uses_arrival_counters(const pa_problem* problem, const pa_tiles* tiles) {
  return !short_path(problem, tiles) && tiles->num_splits > 1 &&
         (tiles->variant & pa::kVariantSeparateMerge) == 0;
}

// pa_decode after its checks: the launches, with the workspace laid out as wl.
pa_status decode_launch(const pa_problem* problem, const pa_tiles* tiles, const void* q,
                        const void* k_pool, const void* v_pool, const int32_t* block_tables,
                        const int32_t* context_lens, void* out, float* lse, void* workspace,
                        const Workspace& wl, hipStream_t stream) {
  pa_status st = PA_OK;
  const int S = tiles->num_splits;
  const int G = problem->num_q_heads / problem->num_kv_heads;
  const int waves = tiles->waves_per_wg;
  const bool even = even_grid(tiles);
  if (problem->num_seqs == 0) return PA_OK;
  if (short_path(problem, tiles))  // G = 32, head dims other than 128, or asked for
    return short_runs(problem, tiles, q, nullptr, k_pool, v_pool, block_tables, context_lens, out,
                      lse, static_cast<char*>(workspace), wl, stream);

  const int ntiles = ceil_div(problem->max_context_len, pa::kDecodeTile);
  pa::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k_pool = static_cast<const uint16_t*>(k_pool);
  p.v_pool = static_cast<const uint16_t*>(v_pool);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.lse = lse;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  p.counters = nullptr;
  p.piece_counts = nullptr;
  p.query_start_loc = nullptr;
  if (S > 1) {
    char* ws = static_cast<char*>(workspace);
    p.part_o = reinterpret_cast<float*>(ws + wl.o_off);
    p.part_lse = reinterpret_cast<float*>(ws + wl.lse_off);
    p.counters = reinterpret_cast<int32_t*>(ws + wl.ctr_off);
    p.piece_counts = reinterpret_cast<int32_t*>(ws + wl.cnt_off);
  }
  p.stride_page = problem->kv_stride_page;
  p.stride_token = problem->kv_stride_token;
  p.stride_head = problem->kv_stride_head;
  p.num_seqs = problem->num_seqs;
  p.num_q_heads = problem->num_q_heads;
  p.num_kv_heads = problem->num_kv_heads;
  p.max_blocks = problem->max_blocks_per_seq;
  p.page_shift = page_shift(problem);
  p.num_splits = even ? S + 1 : S;
  p.tiles_per_split = ntiles > 0 ? ceil_div(ntiles, S) : 1;
  p.max_tiles = ntiles;
  p.even_min_tiles = p.tiles_per_split;
  p.scale_log2 = problem->scale * pa::kLog2eHost;
  p.out_f32 = problem->out_dtype == PA_FP32;
  p.causal = problem->causal;
  const bool separate = S > 1 && (tiles->variant & pa::kVariantSeparateMerge) != 0;
  if (even) {
    const int nw = pa::decode_even_resident(G, waves, stream);
    if (nw <= 0) return PA_ERR_HIP;
    if ((st = from_hip(pa::launch_decode_even(p, G, waves, nw, stream))) != PA_OK) return st;
  } else if ((st = from_hip(pa::launch_decode(p, G, waves, !separate, stream))) != PA_OK) {
    return st;
  }
  if (separate) {
    pa::ReduceParams r;
    r.part_o = p.part_o;
    r.part_lse = p.part_lse;
    r.out = out;
    r.lse = lse;
    r.rows = problem->num_seqs * problem->num_q_heads;
    r.num_splits = p.num_splits;
    r.head_dim = problem->head_dim;
    r.out_f32 = p.out_f32;
    r.query_start_loc = nullptr;
    r.num_q_heads = problem->num_q_heads;
    r.piece_counts = even ? p.piece_counts : nullptr;
    r.context_lens = context_lens;
    r.group = G;
    r.unit_rows = 0;
    // even grid: merge per (sequence, kv head) unit, its G rows in one
    // workgroup, the piece count read once
    st = from_hip(even ? pa::launch_unit_merge(r, problem->num_seqs * problem->num_kv_heads, G,
                                               stream)
                       : pa::launch_reduce(r, stream));
  }
  return st;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape (not built)";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

pa_status pa_workspace_size(const pa_problem* problem, const pa_tiles* tiles,
                            size_t* workspace_bytes) {
  pa_status st = check_attention(problem);
  if (st != PA_OK) return st;
  if ((st = check_tiles(tiles)) != PA_OK) return st;
  if (!workspace_bytes) return PA_ERR_INVALID_ARG;
  *workspace_bytes = workspace_layout(problem, tiles).total;
  return PA_OK;
}

pa_status pa_select_tiles(const pa_problem* problem, pa_tiles* out, size_t* workspace_bytes) {
  pa_status st = check_attention(problem);
  if (st != PA_OK) return st;
  if (!out || !workspace_bytes) return PA_ERR_INVALID_ARG;
  const int G = problem->num_q_heads / problem->num_kv_heads;
  pa_tiles t;
  memset(&t, 0, sizeof t);
  const pa::DecodeChoice dc = pa::table_decode(problem->num_seqs, problem->num_kv_heads,
                                               problem->max_context_len, G);
  if (problem->max_query_len <= 1 && !verify_path(problem)) {
    t.kv_tile = pa::kDecodeTile;
    t.waves_per_wg = dc.waves;
    t.q_tokens_per_tile = 1;
    t.num_splits = dc.splits;
    t.variant = dc.variant;
  } else if (verify_path(problem)) {
    // short query runs: each unit one Q-block of max_query_len tokens x G
    // heads, 4 wavefronts, even-work grid, the short-run split bound
    t.kv_tile = pa::kDecodeTile;
    t.waves_per_wg = 4;
    t.q_tokens_per_tile = problem->max_query_len > 1 ? problem->max_query_len : 1;
    t.num_splits = pa::table_short_splits(problem->num_seqs, problem->num_kv_heads,
                                          problem->max_context_len, problem->head_dim, G,
                                          dc.splits);
    t.variant = (problem->out_dtype == PA_FP32 ? pa::kVariantPreciseP : 0) |
                pa::kVariantSeparateMerge | pa::kVariantEvenWork;
    t.tile_splits = 0;
  } else {
    t.kv_tile = 32;
    t.waves_per_wg = problem->head_dim == 256 ? 4 : 8;
    t.q_tokens_per_tile = query_tile_tokens(problem);
    // single-token sequences of a mixed batch run as split-KV decode work
    t.num_splits = may_hold_decode_rows(problem) ? dc.splits : 1;
    // fp32 outputs ask for more than bf16 weights give: keep P to ~2^-18;
    // single-token sequences take the decode table's grid choice
    t.variant = (problem->out_dtype == PA_FP32 ? pa::kVariantPreciseP : 0) |
                pa::kVariantSeparateMerge | (dc.variant & pa::kVariantEvenWork);
    // Query tiles are not split when single-token sequences run as decode
    // workgroups: measured on gfx950, those already use the CUs that a few
    // long query tiles leave idle, and splitting the tiles then only adds
    // partial traffic (mixed 16 decodes + 2x512-token chunks: 255 us whole,
    // 295 us with two runs per tile; the chunks alone: 197 us -> 134 us).
    // Where single-token sequences are query tiles themselves, their long
    // key runs are split (mixed_tile_splits).
    if (decode_rows_apart(problem)) {
      t.tile_splits = 1;
    } else {
      t.tile_splits = pa::table_prefill_splits(problem->total_query_tokens, t.q_tokens_per_tile,
                                               problem->num_kv_heads, problem->max_context_len,
                                               problem->head_dim);
      if (may_hold_decode_rows(problem))
        t.tile_splits = std::max(t.tile_splits, mixed_tile_splits(problem));
    }
  }
  *out = t;
  return pa_workspace_size(problem, &t, workspace_bytes);
}

pa_status pa_decode(const pa_problem* problem, const pa_tiles* tiles, const void* q,
                    const void* k_pool, const void* v_pool, const int32_t* block_tables,
                    const int32_t* context_lens, void* out, float* lse, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  pa_status st = check_decode(problem, tiles, q, k_pool, v_pool, block_tables, context_lens, out);
  if (st != PA_OK) return st;
  const Workspace wl = workspace_layout(problem, tiles);
  if (wl.dec_total > 0 && (!workspace || workspace_bytes < wl.dec_total ||
                           (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0))
    return PA_ERR_WORKSPACE;
  return decode_launch(problem, tiles, q, k_pool, v_pool, block_tables, context_lens, out, lse,
                       workspace, wl, stream);
}

pa_status pa_decode_noalloc(const pa_problem* problem, const pa_tiles* tiles, const void* q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens, void* out,
                            float* lse, hipStream_t stream) {
  pa_status st = check_decode(problem, tiles, q, k_pool, v_pool, block_tables, context_lens, out);
  if (st != PA_OK) return st;
  const Workspace wl = workspace_layout(problem, tiles);
  if (wl.dec_total > pa::kScratchBytes) return PA_ERR_WORKSPACE;
  if (problem->num_seqs == 0) return PA_OK;
  void* ws = nullptr;
  if (wl.dec_total > 0) {
    ws = pa::scratch_address(stream);
    if (!ws) return PA_ERR_HIP;
    // The array keeps whatever the last call on this GPU left in it; the
    // fused merge's arrival counters are the only values a call reads
    // without writing them first, so they are cleared (a fill kernel, which
    // a graph capture records like any other launch).
    if (uses_arrival_counters(problem, tiles)) {
      const int64_t units = (int64_t)problem->num_seqs * problem->num_kv_heads;
      if ((st = from_hip(pa::launch_zero_words(static_cast<char*>(ws) + wl.ctr_off, units,
                                               stream))) != PA_OK)
        return st;
    }
  }
  return decode_launch(problem, tiles, q, k_pool, v_pool, block_tables, context_lens, out, lse,
                       ws, wl, stream);
}

pa_status pa_prefill(const pa_problem* problem, const pa_tiles* tiles, const void* q,
                     const int32_t* query_start_loc, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* context_lens, void* out,
                     float* lse, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  pa_status st = check_attention(problem);
  if (st != PA_OK) return st;
  if ((st = check_tiles(tiles)) != PA_OK) return st;
  const int G = problem->num_q_heads / problem->num_kv_heads;
  if (!q || !query_start_loc || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PA_ERR_INVALID_ARG;
  // A batch of single-token sequences runs on the decode kernels.  In the
  // unified launch G = 16 has no decode workgroups: its single-token
  // sequences take the prefill tiles.
  const bool decode_only = problem->max_query_len <= 1;
  const bool decode_rows = decode_only || decode_rows_apart(problem);
  const int S = decode_rows ? tiles->num_splits : 1;
  const bool even = decode_rows && even_grid(tiles);
  const int TS = tile_splits_of(problem, tiles);
  const Workspace wl = workspace_layout(problem, tiles);
  if (wl.total > 0 && (!workspace || workspace_bytes < wl.total ||
                       (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0))
    return PA_ERR_WORKSPACE;
  if (problem->num_seqs == 0 || problem->total_query_tokens == 0) return PA_OK;
  if (short_path(problem, tiles))
    return short_runs(problem, tiles, q, query_start_loc, k_pool, v_pool, block_tables,
                      context_lens, out, lse, static_cast<char*>(workspace), wl, stream);
  const int qt = query_tile_tokens(problem);
  const float scale_log2 = problem->scale * pa::kLog2eHost;
  const int out_f32 = problem->out_dtype == PA_FP32;

  pa::PrefillParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.query_start_loc = query_start_loc;
  p.k_pool = static_cast<const uint16_t*>(k_pool);
  p.v_pool = static_cast<const uint16_t*>(v_pool);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.lse = lse;
  p.stride_page = problem->kv_stride_page;
  p.stride_token = problem->kv_stride_token;
  p.stride_head = problem->kv_stride_head;
  p.num_seqs = problem->num_seqs;
  p.num_q_heads = problem->num_q_heads;
  p.num_kv_heads = problem->num_kv_heads;
  p.max_blocks = problem->max_blocks_per_seq;
  p.page_shift = page_shift(problem);
  p.q_tile = qt;
  p.decode_rows_apart = decode_rows ? 1 : 0;
  p.tile_splits = TS;
  p.tpart_o = nullptr;
  p.tpart_lse = nullptr;
  if (TS > 1) {
    char* ws = static_cast<char*>(workspace);
    p.tpart_o = reinterpret_cast<float*>(ws + wl.to_off);
    p.tpart_lse = reinterpret_cast<float*>(ws + wl.tlse_off);
  }
  p.causal = problem->causal;
  p.scale_log2 = scale_log2;
  p.out_f32 = out_f32;

  pa::DecodeParams d;
  d.q = p.q;
  d.k_pool = p.k_pool;
  d.v_pool = p.v_pool;
  d.block_tables = block_tables;
  d.context_lens = context_lens;
  d.out = out;
  d.lse = lse;
  d.part_o = nullptr;
  d.part_lse = nullptr;
  d.counters = nullptr;
  d.query_start_loc = query_start_loc;
  d.piece_counts = nullptr;
  if (S > 1) {
    char* ws = static_cast<char*>(workspace);
    d.part_o = reinterpret_cast<float*>(ws + wl.o_off);
    d.part_lse = reinterpret_cast<float*>(ws + wl.lse_off);
    d.counters = reinterpret_cast<int32_t*>(ws + wl.ctr_off);
    if (even) d.piece_counts = reinterpret_cast<int32_t*>(ws + wl.cnt_off);
  }
  d.stride_page = p.stride_page;
  d.stride_token = p.stride_token;
  d.stride_head = p.stride_head;
  d.num_seqs = problem->num_seqs;
  d.num_q_heads = problem->num_q_heads;
  d.num_kv_heads = problem->num_kv_heads;
  d.max_blocks = problem->max_blocks_per_seq;
  d.page_shift = page_shift(problem);
  d.num_splits = even ? S + 1 : S;
  const int ntiles = ceil_div(problem->max_context_len, pa::kDecodeTile);
  d.tiles_per_split = ntiles > 0 ? ceil_div(ntiles, S) : 1;
  d.max_tiles = ntiles;
  d.even_min_tiles = d.tiles_per_split;
  d.scale_log2 = scale_log2;
  d.out_f32 = out_f32;
  d.causal = problem->causal;

  // an LSE is asked for: weights as bf16 high part + remainder, so its
  // denominator is not rounded to bf16's 8-bit significand
  const bool precise = (tiles->variant & pa::kVariantPreciseP) != 0 || lse != nullptr;
  if (decode_only) {
    // every sequence is a decode row: the decode kernels alone (measured on a
    // batch of 64: 231 us against 267 us for the decode part of the unified
    // kernel, whose registers allow one 512-thread workgroup per CU); splits
    // are always merged by the separate kernel here
    const int waves = tiles->waves_per_wg;
    if (waves != 4 && waves != 8) return PA_ERR_INVALID_ARG;
      if (even) {
      const int nw = pa::decode_even_resident(G, waves, stream);
      if (nw <= 0) return PA_ERR_HIP;
      if ((st = from_hip(pa::launch_decode_even(d, G, waves, nw, stream))) != PA_OK) return st;
    } else if ((st = from_hip(pa::launch_decode(d, G, waves, false, stream))) != PA_OK) {
      return st;
    }
    if (S > 1) {
      pa::ReduceParams r;
      r.part_o = d.part_o;
      r.part_lse = d.part_lse;
      r.out = out;
      r.lse = lse;
      r.rows = problem->num_seqs * problem->num_q_heads;
      r.num_splits = d.num_splits;
      r.head_dim = problem->head_dim;
      r.out_f32 = out_f32;
      r.query_start_loc = query_start_loc;
      r.num_q_heads = problem->num_q_heads;
      r.piece_counts = d.piece_counts;
      r.context_lens = context_lens;
      r.group = G;
      r.unit_rows = 0;
      st = from_hip(pa::launch_reduce(r, stream));
    }
    return st;
  }
  // static grid: sum over sequences of ceil(q_len / qt) <= ceil(T / qt) + B
  const int64_t nx = (int64_t)ceil_div(problem->total_query_tokens, qt) + problem->num_seqs;
  int64_t n_dec = decode_rows ? (int64_t)problem->num_seqs * problem->num_kv_heads * S : 0;
  if (even) {
    n_dec = pa::unified_resident(G, precise, problem->head_dim, stream);
    if (n_dec <= 0) return PA_ERR_HIP;
  }
  if (nx * problem->num_kv_heads * TS + n_dec > 0x7fffffff) return PA_ERR_UNSUPPORTED;
  if ((st = from_hip(pa::launch_prefill(p, d, G, (int)nx, (int)n_dec, precise, problem->head_dim,
                                        stream))) != PA_OK)
    return st;
  if (TS > 1) {
    pa::TileMergeParams m;
    m.tpart_o = p.tpart_o;
    m.tpart_lse = p.tpart_lse;
    m.query_start_loc = query_start_loc;
    m.out = out;
    m.lse = lse;
    m.num_seqs = problem->num_seqs;
    m.num_q_heads = problem->num_q_heads;
    m.num_kv_heads = problem->num_kv_heads;
    m.q_tile = qt;
    m.decode_rows_apart = p.decode_rows_apart;
    m.tile_splits = TS;
    m.out_f32 = out_f32;
    if ((st = from_hip(pa::launch_tile_merge(m, (int)nx, problem->head_dim, stream))) != PA_OK)
      return st;
  }
  if (decode_rows && S > 1) {
    pa::ReduceParams r;
    r.part_o = d.part_o;
    r.part_lse = d.part_lse;
    r.out = out;
    r.lse = lse;
    r.rows = problem->num_seqs * problem->num_q_heads;
    r.num_splits = d.num_splits;
    r.head_dim = problem->head_dim;
    r.out_f32 = out_f32;
    r.query_start_loc = query_start_loc;
    r.num_q_heads = problem->num_q_heads;
    r.piece_counts = d.piece_counts;
    r.context_lens = context_lens;
    r.group = G;
    r.unit_rows = 0;
    // The decode workgroups write their partials at sequence rows b*Hq + h,
    // and only single-token sequences own any: the per-row merge maps each
    // such row to its token's output row and skips every other sequence
    // before it reads a piece count (which may be stale for them).
    st = from_hip(pa::launch_reduce(r, stream));
  }
  return st;
}

pa_status pa_cache_append(const pa_problem* problem, const void* k_new, const void* v_new,
                          const int32_t* query_start_loc, const int32_t* block_tables,
                          const int32_t* context_lens, void* k_pool, void* v_pool,
                          hipStream_t stream) {
  pa_status st = check_problem(problem);
  if (st != PA_OK) return st;
  if (!k_new || !v_new || !block_tables || !context_lens || !k_pool || !v_pool)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return PA_ERR_INVALID_ARG;
  if (!query_start_loc && problem->total_query_tokens != problem->num_seqs)
    return PA_ERR_INVALID_ARG;  // one token per sequence
  if (problem->num_seqs == 0 || problem->total_query_tokens == 0) return PA_OK;
  pa::AppendParams p;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.query_start_loc = query_start_loc;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.k_pool = static_cast<uint16_t*>(k_pool);
  p.v_pool = static_cast<uint16_t*>(v_pool);
  p.stride_page = problem->kv_stride_page;
  p.stride_token = problem->kv_stride_token;
  p.stride_head = problem->kv_stride_head;
  p.num_seqs = problem->num_seqs;
  p.num_kv_heads = problem->num_kv_heads;
  p.max_blocks = problem->max_blocks_per_seq;
  p.log2_page = log2_page(problem);
  p.total_tokens = problem->total_query_tokens;
  p.head_dim = problem->head_dim;
  return from_hip(pa::launch_append(p, stream));
}

pa_status pa_check_inputs(const pa_problem* problem, int64_t num_pages,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start_loc, int32_t* flags, hipStream_t stream) {
  pa_status st = check_problem(problem);
  if (st != PA_OK) return st;
  if (!block_tables || !context_lens || !flags || num_pages <= 0) return PA_ERR_INVALID_ARG;
  if (!query_start_loc && problem->total_query_tokens != problem->num_seqs)
    return PA_ERR_INVALID_ARG;  // one token per sequence
  pa::CheckParams p;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start_loc = query_start_loc;
  p.flags = flags;
  p.num_pages = num_pages;
  p.num_seqs = problem->num_seqs;
  p.max_blocks = problem->max_blocks_per_seq;
  p.log2_page = log2_page(problem);
  p.max_context_len = problem->max_context_len;
  p.max_query_len = query_start_loc ? problem->max_query_len : 1;
  p.total_tokens = problem->total_query_tokens;
  p.chunks = ceil_div(problem->max_blocks_per_seq, 256);
  return from_hip(pa::launch_check(p, stream));
}

pa_status pa_splitkv_reduce(const float* partial_o, const float* partial_lse, int32_t rows,
                            int32_t num_splits, int32_t head_dim, void* out,
                            pa_dtype out_dtype, float* lse_out, hipStream_t stream) {
  if (rows < 0 || num_splits < 1 || num_splits > pa::kReduceMaxSplits || head_dim <= 0 ||
      head_dim % 4 != 0 || head_dim > 1024)
    return PA_ERR_INVALID_ARG;
  if (!dtype_valid(out_dtype)) return PA_ERR_INVALID_ARG;
  if (rows == 0) return PA_OK;
  if (!partial_o || !partial_lse || !out) return PA_ERR_INVALID_ARG;
  if (!aligned16(partial_o) || !aligned16(out)) return PA_ERR_INVALID_ARG;
  pa::ReduceParams r;
  r.part_o = partial_o;
  r.part_lse = partial_lse;
  r.out = out;
  r.lse = lse_out;
  r.rows = rows;
  r.num_splits = num_splits;
  r.head_dim = head_dim;
  r.out_f32 = out_dtype == PA_FP32;
  r.query_start_loc = nullptr;
  r.num_q_heads = 1;
  r.piece_counts = nullptr;
  r.context_lens = nullptr;
  r.group = 1;
  r.unit_rows = 0;
  return from_hip(pa::launch_reduce(r, stream));
}

}  // extern "C"
