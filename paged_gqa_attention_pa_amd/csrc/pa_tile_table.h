// Launch-shape table: the runtime only looks shapes up here, it never tunes
// (the offline micro-benchmark + decision-table idea of the IBM Triton
// summary, section on moving autotuning offline).  The decode rule comes from
// sweeps on gfx950 (batch 1 and 8 at contexts 4k-256k, batch 64 at 4k-8k):
// the kernel streams at its best with at least ~256 workgroups in the grid
// and at most 64 tiles (1024 keys) per workgroup, which bounds the tail of
// the longest sequence; fewer, larger splits also keep the merge cheap.
#pragma once

#include <stdint.h>

namespace pa {

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
  return group >= 16 ? 4 : 4;
}

// Decode variant bits (pa_tiles.variant).  Merging the splits in a second
// kernel measured faster than the last-workgroup merge at every size tried
// on gfx950 (the agent-scope release each split needs writes back the L2).
inline int table_decode_variant(int num_seqs, int num_kv_heads, int max_context_len) {
  (void)num_seqs;
  (void)num_kv_heads;
  (void)max_context_len;
  return 2;
}

}  // namespace pa
