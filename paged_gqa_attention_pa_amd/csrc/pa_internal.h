// Internal interface between the C-ABI host code and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kHeadDim = 128;   // built head dimension
constexpr int kPage = 16;       // keys per block of the prefill page window; smallest page size
constexpr int kDecodeTile = 16; // keys per decode step (one MFMA N-tile)
constexpr int kMaxSplits = 256;        // decode split-KV
constexpr int kReduceMaxSplits = 4096; // pa_splitkv_reduce
constexpr int kMaxTileSplits = 8;      // prefill: splits of one query tile's keys
constexpr float kLog2eHost = 1.4426950408889634f;
// Bytes of the per-device scratch array behind pa_decode_noalloc.
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;

// pa_tiles.variant bits
constexpr int kVariantPreciseP = 1;      // prefill: P as bf16 high + remainder
constexpr int kVariantSeparateMerge = 2; // decode: merge splits in a second kernel
constexpr int kVariantEvenWork = 4;      // decode: even-work grid (with the separate merge)
constexpr int kVariantShortDecode = 8;   // decode: rows on the short-run kernel (even grid)

struct DecodeParams {
  const uint16_t* q;        // [B, Hq, D] bf16
  const uint16_t* k_pool;   // paged pools, bf16
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;                // [B, Hq, D] bf16 or fp32
  float* lse;               // [B, Hq] or null
  float* part_o;            // [B*Hq, S, D] when S > 1
  float* part_lse;          // [B*Hq, S]
  int32_t* counters;        // [B*Hkv] split arrival counters, zero between calls
  const int32_t* query_start_loc;  // mixed batch: [B+1]; null for a pure decode batch
  int64_t stride_page, stride_token, stride_head;
  int32_t num_seqs, num_q_heads, num_kv_heads, max_blocks;
  int32_t page_shift;       // log2(page_size / 16): 16-key tiles per page = 1 << page_shift
  int32_t tiles_per_split;  // 16-key tiles per split
  int32_t num_splits;       // partial slots per row (even-work grid: splits + 1)
  int32_t max_tiles;        // ceil(max_context_len / 16): bound on a unit's tiles
  int32_t even_min_tiles;   // even-work grid: least tiles per workgroup
  int32_t* piece_counts;    // even-work grid: [B*Hkv] pieces per unit
  float scale_log2;         // scale * log2(e)
  int32_t out_f32;
  int32_t causal;           // short query runs: causal within the run
};

struct PrefillParams {
  const uint16_t* q;        // [T, Hq, D] bf16
  const int32_t* query_start_loc;  // [B+1]
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;                // [T, Hq, D]
  float* lse;               // [T, Hq] or null
  int64_t stride_page, stride_token, stride_head;
  int32_t num_seqs, num_q_heads, num_kv_heads, max_blocks;
  int32_t page_shift;       // log2(page_size / 16)
  int32_t q_tile;           // query tokens per workgroup
  int32_t decode_rows_apart;  // 1: single-token sequences run as decode workgroups
  // tile_splits > 1: each query tile's key range is cut into that many runs
  // of whole 32-key tiles, one workgroup each, writing normalised partials
  // (fp32, [T*Hq, tile_splits, D]) and their lse ([T*Hq, tile_splits],
  // natural log) instead of out / lse; tile_merge_kernel combines them.
  int32_t tile_splits;
  float* tpart_o;
  float* tpart_lse;
  int32_t causal;
  float scale_log2;
  int32_t out_f32;
};

struct ReduceParams {
  const float* part_o;      // [rows, S, D]
  const float* part_lse;    // [rows, S]
  void* out;                // [rows, D]
  float* lse;               // [rows] or null
  int32_t rows, num_splits, head_dim, out_f32;
  // Mixed batch: rows are (sequence, q head) pairs, only single-token
  // sequences are merged, into output row query_start_loc[s]*Hq + h.
  const int32_t* query_start_loc;  // null: output row = partial row
  int32_t num_q_heads;
  // Even-work decode grid: row (b, h) has piece_counts[b*Hkv + h/G] slots
  // in use (rows of one piece were written directly and are skipped; rows of
  // an empty context get O = 0, lse = -inf).  Null: every slot is in use.
  const int32_t* piece_counts;
  const int32_t* context_lens;
  int32_t group;
  // Short-run partials (rows are (token, q head) pairs): > 0 launches a
  // (units, unit_rows) grid, workgroup (u, r) merging row r of unit u =
  // (sequence, kv head), token r / G of the sequence (query_start_loc, or
  // token u / Hkv when it is null), head (u % Hkv) * G + r % G.
  int32_t unit_rows;
};

// Merge of split query tiles: one workgroup per (query tile, kv head) of the
// prefill grid, without the split index.
struct TileMergeParams {
  const float* tpart_o;     // [T*Hq, S, D]
  const float* tpart_lse;   // [T*Hq, S]
  const int32_t* query_start_loc;  // [B+1]
  void* out;                // [T, Hq, D]
  float* lse;               // [T, Hq] or null
  int32_t num_seqs, num_q_heads, num_kv_heads;
  int32_t q_tile, decode_rows_apart, tile_splits, out_f32;
};

struct AppendParams {
  const uint16_t* k_new;    // [T, Hkv, D] bf16
  const uint16_t* v_new;
  const int32_t* query_start_loc;  // [B+1] or null (row t = sequence t)
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint16_t* k_pool;
  uint16_t* v_pool;
  int64_t stride_page, stride_token, stride_head;
  int32_t num_seqs, num_kv_heads, max_blocks, total_tokens;
  int32_t head_dim;         // 64, 128 or 256
  int32_t log2_page;        // log2(page_size)
};

// Launchers: return hipSuccess or the launch error.  Shapes were checked.
hipError_t launch_decode(const DecodeParams& p, int group, int waves, bool fused,
                         hipStream_t stream);
// Even-work decode grid of nw workgroups (separate merge only).
hipError_t launch_decode_even(const DecodeParams& p, int group, int waves, int nw,
                              hipStream_t stream);
// Device that work enqueued on `stream` runs on (the current device for the
// null stream), or -1.  The occupancy figures below are cached per device,
// keyed on it.
int stream_device(hipStream_t stream);
// Workgroups of the even-work decode kernel that fit at once on the device
// of `stream`.
int decode_even_resident(int group, int waves, hipStream_t stream);
// Prefill tiles (nx x Hkv workgroups) and n_dec decode workgroups (split x
// Hkv x B, for the single-token sequences of a mixed batch) in one launch.
hipError_t launch_prefill(const PrefillParams& pp, const DecodeParams& dp, int group, int nx,
                          int n_dec, bool precise_p, int head_dim, hipStream_t stream);
// Workgroups of the unified prefill kernel that fit at once on the device of
// `stream`.
int unified_resident(int group, bool precise_p, int head_dim, hipStream_t stream);
hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream);

// pa_check_inputs: device-side checks of the tables and lengths.
struct CheckParams {
  const int32_t* block_tables;     // [B, max_blocks]
  const int32_t* context_lens;     // [B]
  const int32_t* query_start_loc;  // [B+1] or null (one token per sequence)
  int32_t* flags;                  // device int32, PA_CHECK_* bits
  int64_t num_pages;
  int32_t num_seqs, max_blocks, max_context_len, max_query_len, total_tokens;
  int32_t log2_page;               // log2(page_size)
  int32_t chunks;                  // ceil(max_blocks / 256): workgroups per sequence
};
// Clears *flags, then ORs in the PA_CHECK_* bit of every failed check.
hipError_t launch_check(const CheckParams& p, hipStream_t stream);
// Short-run path: merge the pieces of every (sequence, kv head) unit (rows
// are (token, q head) pairs; piece_counts and context_lens are required,
// query_start_loc null means one token per sequence); units = num_seqs *
// num_kv_heads, unit_rows = the longest run's rows (max_query_len * G).
// Many rows merge with one workgroup per unit, few with one per (unit, row).
hipError_t launch_unit_merge(const ReduceParams& p, int units, int unit_rows,
                             hipStream_t stream);
// Short query runs (1 <= q_s, q_s * G <= 64; <= 32 at head dim 256): 16-row
// blocks per unit (1, 2 or 4; 0 when not built), resident workgroups of that
// kernel, and the even-work launch of nw workgroups.
int verify_row_blocks(int group, int max_query_len, int head_dim);
int verify_resident(int group, int rb, bool precise_p, int head_dim, hipStream_t stream);
hipError_t launch_verify(const DecodeParams& p, int group, int rb, bool precise_p, int head_dim,
                         int nw, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
// pa_decode_noalloc's scratch array: its device address on the device of
// `stream` (looked up once per device), or null on failure.
void* scratch_address(hipStream_t stream);
// Zero `words` 32-bit words at p with a fill kernel on `stream`.
hipError_t launch_zero_words(void* p, int64_t words, hipStream_t stream);
hipError_t launch_tile_merge(const TileMergeParams& p, int nx, int head_dim, hipStream_t stream);

}  // namespace pa
