// The even-work grid driver shared by the decode and short-run kernels.
#pragma once

#include "pa_decode_body.h"
#include "pa_even_plan.h"
#include "pa_verify_body.h"

namespace pa {
namespace decode_detail {

// Even-work grid (for batches whose context lengths differ).  The decode
// tiles of all (sequence, kv head) units are laid end to end, units ordered
// by sequence then kv head, a unit of sequence b being n_b = ceil(L_b / 16)
// tiles (0 for a sequence that is not a single-token row of a mixed batch):
// N = Hkv * sum_b n_b tiles.  Workgroup w of nw takes tiles
// [w*Wt, min((w+1)*Wt, N)), Wt = max(min_tiles, ceil(N / nw)), so every
// workgroup streams the same number of tiles whatever the length mix; a
// static (split, head, sequence) grid leaves the CUs that drew long
// sequences running alone at the end.  A unit of at most max_tiles tiles
// meets at most ceil(max_tiles / min_tiles) + 1 <= num_splits workgroups, one
// partial slot each (slot = workgroup - first workgroup of the unit); a unit
// inside one workgroup is written to the output directly.  The workgroup that
// holds a unit's last tile records its piece count for the merge.
//
// RB = 0: units of single-token sequences, decode_body.  RB >= 1: units of
// sequences with 1 <= q_s and q_s * G <= 16 * RB query tokens, verify_body
// (every unit is then a row block of the short-run Q-block).
template <int G, int W, int RB = 0, bool PRECISE = false, int D = kHeadDim>
__device__ void decode_even_body(const DecodeParams& p, int w, int nw, float* sm_buf) {
  constexpr int kT = 64 * W;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ long long s_part[W];
  __shared__ long long s_start;  // sum of n_b over sequences before s_seq
  __shared__ int s_seq;
  const int B = p.num_seqs, Hkv = p.num_kv_heads;
  auto seq_tiles = [&](int b) -> int {
    if constexpr (RB == 0) {
      if (p.query_start_loc && p.query_start_loc[b + 1] - p.query_start_loc[b] != 1) return 0;
    } else {
      const int qn = p.query_start_loc ? p.query_start_loc[b + 1] - p.query_start_loc[b] : 1;
      if (qn <= 0 || qn * G > 16 * RB) return 0;
    }
    const int L = p.context_lens[b];
    return min((L + kDecodeTile - 1) / kDecodeTile, min(p.max_blocks << p.page_shift, p.max_tiles));
  };
  // Pass 1: total tiles.
  long long tot = 0;
  for (int b = tid; b < B; b += kT) tot += seq_tiles(b);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
  if (lane == 0) s_part[wave] = tot;
  __syncthreads();
  long long per_head = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) per_head += s_part[i];
  const long long N = per_head * Hkv;
  if (N == 0) return;
  const long long Wt = even_plan::tiles_per_workgroup(N, nw, p.even_min_tiles);
  const long long R0 = (long long)w * Wt;
  if (R0 >= N) return;
  const long long R1 = R0 + Wt < N ? R0 + Wt : N;

  // Pass 2: the sequence holding tile R0 (prefix sums, 64W sequences a step).
  if (tid == 0) s_seq = -1;
  long long base = 0;
  for (int c0 = 0; c0 < B; c0 += kT) {
    const int b = c0 + tid;
    const int nb = b < B ? seq_tiles(b) : 0;
    long long v = nb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    __syncthreads();
    if (lane == 63) s_part[wave] = v;
    __syncthreads();
    long long wbase = 0, chunk = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if (i < wave) wbase += s_part[i];
      chunk += s_part[i];
    }
    const long long incl = base + wbase + v;  // sum of n over sequences <= b
    if (nb > 0 && (incl - nb) * Hkv <= R0 && R0 < incl * Hkv) {
      s_seq = b;
      s_start = incl - nb;
    }
    base += chunk;
    __syncthreads();
    if (s_seq >= 0) break;
  }
  even_plan::Cursor cur{R0, s_start, s_seq, seq_tiles(s_seq)};
  const int S = p.num_splits;  // partial slots per row
  while (true) {
    const even_plan::Piece pc = even_plan::piece_at(cur, R1, Wt, Hkv, w);
    const int b = cur.b;
    const EvenPiece piece{pc.t0, pc.t1, pc.slot, S, pc.direct};
    if constexpr (RB == 0)
      decode_body<G, W, false, true>(p, 0, pc.g, b, sm_buf, piece);
    else
      verify_detail::verify_body<G, RB, W, PRECISE, D>(p, pc.g, b, sm_buf, piece);
    if (tid == 0 && pc.last) p.piece_counts[(int64_t)b * Hkv + pc.g] = pc.pieces;
    __syncthreads();  // the next piece reuses the LDS merge buffers
    cur.pos += pc.t1 - pc.t0;
    if (cur.pos >= R1) break;
    if (even_plan::ends_sequence(pc, cur.nb, Hkv)) {  // next sequence with tiles
      cur.P += cur.nb;
      do {
        ++cur.b;
        cur.nb = seq_tiles(cur.b);
      } while (cur.nb == 0);
    }
  }
}

}  // namespace decode_detail
}  // namespace pa
