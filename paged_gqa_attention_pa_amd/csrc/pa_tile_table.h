// Launch-shape table: the runtime only looks shapes up here, it never tunes
// (the offline micro-benchmark + decision-table idea of the IBM Triton
// summary, section on moving autotuning offline).  The decode rule comes from
// sweeps on gfx950 (batch 1 and 8 at contexts 4k-256k, batch 64 at 4k-8k):
// the kernel streams at its best with at least ~256 workgroups in the grid
// and at most 64 tiles (1024 keys) per workgroup, which bounds the tail of
// the longest sequence; fewer, larger splits also keep the merge cheap.
#pragma once

#include <stdint.h>

#include "pa_tile_table_gen.h"

namespace pa {

// Fallback rules below cover shapes outside the swept buckets.

inline int table_decode_splits(int num_seqs, int num_kv_heads, int max_context_len) {
  const int64_t ntiles = (max_context_len + 15) / 16;
  if (ntiles <= 4 || num_seqs <= 0) return 1;
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  int64_t s_par = (256 + units - 1) / units;  // fill the chip
  int64_t s_bal = (ntiles + 63) / 64;         // <= 64 tiles per workgroup
  int64_t splits = s_par > s_bal ? s_par : s_bal;
  const int64_t s_cap = ntiles / 4;           // >= 4 tiles (one per wave) per split
  if (splits > s_cap) splits = s_cap;
  if (splits > 256) splits = 256;
  return splits < 1 ? 1 : (int)splits;
}

inline int table_decode_waves(int num_seqs, int num_kv_heads, int max_context_len, int group) {
  (void)num_seqs;
  (void)num_kv_heads;
  (void)max_context_len;
  (void)group;
  return 4;
}

// Decode variant bits (pa_tiles.variant).  Merging the splits in a second
// kernel measured faster than the last-workgroup merge at every size tried
// on gfx950 (the agent-scope release each split needs writes back the L2).
// With more than one sequence, lengths may differ: the even-work grid
// (variant bit 2) gives every workgroup the same number of tiles.  Measured
// on a batch of 64 with contexts U[128, 8192]: the static grid streams at
// 3.8 TB/s, equal lengths of the same total at 5.2 TB/s.
inline int table_decode_variant(int num_seqs, int num_kv_heads, int max_context_len) {
  (void)num_kv_heads;
  (void)max_context_len;
  return num_seqs > 1 ? 2 | 4 : 2;
}

// Prefill: how many runs each query tile's keys are cut into.  A query tile
// is one 512-thread workgroup that keeps a CU's matrix cores busy, and a
// mixed batch's decode workgroups stream alongside it, so the aim is about
// one tile workgroup per CU (256): a chunked prefill of thousands of tokens
// needs no split, two 512-token chunks on long prefixes need two runs per
// tile.  Runs shorter than 16 key tiles (512 keys) are not worth their
// partials.  prefill_tokens is the host's bound on tokens that form tiles.
inline int table_prefill_tile_splits(int64_t prefill_tokens, int q_tile, int num_kv_heads,
                                     int max_context_len) {
  if (prefill_tokens <= 0 || q_tile <= 0) return 1;
  const int64_t wgs = (prefill_tokens + q_tile - 1) / q_tile * num_kv_heads;
  int64_t s = 256 / wgs;
  const int64_t s_keys = max_context_len / 512;
  if (s > s_keys) s = s_keys;
  if (s > 8) s = 8;
  return s < 1 ? 1 : (int)s;
}

// Index of the first bucket >= v, or -1 past the last one.
template <int N>
inline int bucket_of(const int (&buckets)[N], int64_t v) {
  for (int i = 0; i < N; ++i)
    if (v <= buckets[i]) return i;
  return -1;
}

// Index of the last bucket <= v (0 below the first).  Units round down: a
// batch with fewer (sequence, kv head) units than a bucket wants at least
// that bucket's split count, never fewer.
template <int N>
inline int bucket_floor(const int (&buckets)[N], int64_t v) {
  int i = 0;
  while (i + 1 < N && buckets[i + 1] <= v) ++i;
  return i;
}

struct DecodeChoice {
  int splits, waves, variant;
};

// Index of the last entry <= v of an ascending list (0 below the first).
template <int N>
inline int index_floor(const int (&vals)[N], int v) {
  int i = 0;
  while (i + 1 < N && vals[i + 1] <= v) ++i;
  return i;
}

// Decode launch shape: the swept entry for the (G, units, context-bound)
// bucket when there is one (G rounded down to a swept group), else the
// fallback rules.
inline DecodeChoice table_decode(int num_seqs, int num_kv_heads, int max_context_len,
                                 int group) {
  DecodeChoice c{table_decode_splits(num_seqs, num_kv_heads, max_context_len),
                 table_decode_waves(num_seqs, num_kv_heads, max_context_len, group),
                 table_decode_variant(num_seqs, num_kv_heads, max_context_len)};
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  const int ui = units > 2 * gen::kUnitBuckets[sizeof(gen::kUnitBuckets) / sizeof(int) - 1]
                     ? -1
                     : bucket_floor(gen::kUnitBuckets, units);
  const int ci = bucket_of(gen::kCtxBuckets, max_context_len);
  const int gi = index_floor(gen::kDecodeGroups, group);
  if (ui >= 0 && ci >= 0 && gen::kDecode[gi][ui][ci][0] > 0) {
    c.splits = gen::kDecode[gi][ui][ci][0];
    c.waves = gen::kDecode[gi][ui][ci][1];
    c.variant = gen::kDecode[gi][ui][ci][2];
  }
  if (c.splits <= 1) {
    c.splits = 1;
    c.variant = 2;
  }
  return c;
}

// Short query runs (one Q-block per (sequence, kv head) unit): the swept split
// bound for the (head dim, G >= 16) key and (units, context-bound) bucket
// when there is one, else the decode choice, whose grid it shares.
inline int table_short_splits(int num_seqs, int num_kv_heads, int max_context_len, int head_dim,
                              int group, int decode_splits) {
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  constexpr int kLast = sizeof(gen::kShortUnitBuckets) / sizeof(int) - 1;
  const int ui = units > 2 * gen::kShortUnitBuckets[kLast]
                     ? -1
                     : bucket_floor(gen::kShortUnitBuckets, units);
  const int ci = bucket_of(gen::kShortCtxBuckets, max_context_len);
  int ki = -1;
  constexpr int kKeys = sizeof(gen::kShortKeys) / sizeof(gen::kShortKeys[0]);
  for (int k = 0; k < kKeys; ++k)
    if (gen::kShortKeys[k][0] == head_dim && gen::kShortKeys[k][1] == (group >= 16 ? 1 : 0))
      ki = k;
  if (ki >= 0 && ui >= 0 && ci >= 0 && gen::kShortSplits[ki][ui][ci] > 0)
    return gen::kShortSplits[ki][ui][ci];
  return decode_splits;
}

// Prefill tile_splits from the sweep of batches of query tiles (swept without
// single-token sequences; pa_select_tiles raises it for mixed batches whose
// single-token sequences run as query tiles).
inline int table_prefill_splits(int64_t total_query_tokens, int q_tile, int num_kv_heads,
                                 int max_context_len, int head_dim) {
  const int64_t wgs = (total_query_tokens + q_tile - 1) / q_tile * num_kv_heads;
  const int wi = bucket_of(gen::kPfWgBuckets, wgs);
  const int ci = bucket_of(gen::kPfCtxBuckets, max_context_len);
  int di = -1;
  constexpr int kDims = sizeof(gen::kPfDims) / sizeof(int);
  for (int k = 0; k < kDims; ++k)
    if (gen::kPfDims[k] == head_dim) di = k;
  if (di >= 0 && wi >= 0 && ci >= 0 && gen::kPrefillTileSplits[di][wi][ci] > 0)
    return gen::kPrefillTileSplits[di][wi][ci];
  return table_prefill_tile_splits(total_query_tokens, q_tile, num_kv_heads, max_context_len);
}

}  // namespace pa
