// Launch-shape table: the runtime only looks shapes up here, it never tunes
// (the offline micro-benchmark + decision-table idea of the IBM Triton
// summary, section on moving autotuning offline).  Until a sweep on gfx950
// fills it, the decode split count follows one rule: give each workgroup
// about max(4, total 16-key tiles / 2048) tiles, at most 128 splits.
#pragma once

#include <stdint.h>

namespace pa {

inline int table_decode_splits(int num_seqs, int num_kv_heads, int max_context_len) {
  const int64_t ntiles = (max_context_len + 15) / 16;
  if (ntiles <= 4 || num_seqs <= 0) return 1;
  int64_t tps = ((int64_t)num_seqs * num_kv_heads * ntiles + 2047) / 2048;
  if (tps < 4) tps = 4;
  if (tps > 64) tps = 64;
  int64_t splits = (ntiles + tps - 1) / tps;
  if (splits > 128) splits = 128;
  return splits < 1 ? 1 : (int)splits;
}

}  // namespace pa
