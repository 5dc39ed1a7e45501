// CPU replay of the even-work grid's partition: every workgroup's walk, with
// the arithmetic the kernels use (pa_even_plan.h), over seeded random length
// mixes.  Checks that every tile of every (sequence, kv head) unit is taken
// exactly once, that partial slots stay below num_splits + 1, that the piece
// count the last workgroup records equals the workgroups that took a piece of
// the unit and that their slots are 0..pieces-1, and that a unit is written
// directly exactly when it is one piece.  The scan that finds a workgroup's
// first sequence is a serial prefix sum here (a parallel one on the GPU).
//
// Usage: even_plan_replay CASES SEED; prints "OK ..." or the first failure
// and exits non-zero.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <vector>

#include "../paged_gqa_attention_pa_amd/csrc/pa_even_plan.h"

namespace {

uint64_t g_state;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
int uniform(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }

int fail(const char* what, int cs, int w, int b, int g) {
  std::printf("FAIL case %d: %s (workgroup %d, sequence %d, kv head %d)\n", cs, what, w, b, g);
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 300;
  g_state = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1;
  long long total_pieces = 0;
  for (int cs = 0; cs < cases; ++cs) {
    const int B = uniform(1, 300);
    static const int kHeads[] = {1, 2, 8, 8};
    const int Hkv = kHeads[uniform(0, 3)];
    const int S = uniform(1, 256);  // the caller's split count: S + 1 slots per row
    const int nw = uniform(1, 2048);
    const int kind = uniform(0, 3);
    std::vector<int> L(B);
    int max_ctx = 0;
    for (int b = 0; b < B; ++b) {
      if (kind == 0) L[b] = uniform(0, 40000);                     // wide spread
      else if (kind == 1) L[b] = uniform(0, 3) == 0 ? 0 : uniform(1, 17);  // tiny, empty
      else if (kind == 2) L[b] = 8192;                              // equal
      else L[b] = uniform(0, 1) ? uniform(128, 8192) : uniform(0, 200000);
      if (L[b] > max_ctx) max_ctx = L[b];
    }
    max_ctx += uniform(0, 100);  // the host bound may exceed every length
    const int max_tiles = (max_ctx + 15) / 16;
    // pages of 16 << ps slots; the table may hold more entries than needed,
    // or (a context past the table, which the input checks report) fewer
    const int ps = uniform(0, 3) == 0 ? uniform(1, 6) : 0;
    const int need = (max_tiles + (1 << ps) - 1) >> ps;
    const int max_blocks = std::max(1, need + uniform(-1, 3));
    const long long min_tiles = max_tiles > 0 ? (max_tiles + S - 1) / S : 1;
    const int slots = S + 1;
    // tiles per sequence, as the kernels clamp them
    std::vector<int> nt(B);
    long long per_head = 0;
    for (int b = 0; b < B; ++b) {
      const int t = (L[b] + 15) / 16;
      const int cap = (max_blocks << ps) < max_tiles ? (max_blocks << ps) : max_tiles;
      nt[b] = t < cap ? t : cap;
      per_head += nt[b];
    }
    const long long N = per_head * Hkv;
    if (N == 0) continue;
    const long long Wt = pa::even_plan::tiles_per_workgroup(N, nw, min_tiles);
    // coverage[b][g][t], slots seen, recorded counts
    std::vector<std::vector<std::vector<int>>> cov(B);
    std::vector<std::vector<std::vector<int>>> seen_slots(B);
    std::vector<std::vector<int>> recorded(B), direct_seen(B);
    for (int b = 0; b < B; ++b) {
      cov[b].assign(Hkv, std::vector<int>(nt[b], 0));
      seen_slots[b].assign(Hkv, std::vector<int>());
      recorded[b].assign(Hkv, -1);
      direct_seen[b].assign(Hkv, -1);
    }
    for (int w = 0; w < nw; ++w) {
      const long long R0 = (long long)w * Wt;
      if (R0 >= N) break;
      const long long R1 = R0 + Wt < N ? R0 + Wt : N;
      // first sequence: (incl - nb) * Hkv <= R0 < incl * Hkv
      long long incl = 0;
      int b0 = -1;
      long long start = 0;
      for (int b = 0; b < B; ++b) {
        incl += nt[b];
        if (nt[b] > 0 && (incl - nt[b]) * Hkv <= R0 && R0 < incl * Hkv) {
          b0 = b;
          start = incl - nt[b];
          break;
        }
      }
      if (b0 < 0) return fail("no sequence holds the first tile", cs, w, -1, -1);
      pa::even_plan::Cursor cur{R0, start, b0, nt[b0]};
      long long taken = 0;
      while (true) {
        const pa::even_plan::Piece p = pa::even_plan::piece_at(cur, R1, Wt, Hkv, w);
        const int b = cur.b;
        if (p.g < 0 || p.g >= Hkv) return fail("kv head out of range", cs, w, b, p.g);
        if (p.t0 < 0 || p.t1 > cur.nb || p.t1 <= p.t0) return fail("bad tile range", cs, w, b, p.g);
        if (p.slot < 0 || p.slot >= slots) return fail("slot past num_splits + 1", cs, w, b, p.g);
        for (int t = p.t0; t < p.t1; ++t) cov[b][p.g][t]++;
        seen_slots[b][p.g].push_back(p.slot);
        if (direct_seen[b][p.g] >= 0 && direct_seen[b][p.g] != (int)p.direct)
          return fail("pieces of one unit disagree on direct", cs, w, b, p.g);
        direct_seen[b][p.g] = p.direct;
        if (p.last) {
          if (recorded[b][p.g] >= 0) return fail("two workgroups record a count", cs, w, b, p.g);
          recorded[b][p.g] = p.pieces;
        }
        ++total_pieces;
        taken += p.t1 - p.t0;
        cur.pos += p.t1 - p.t0;
        if (cur.pos >= R1) break;
        if (pa::even_plan::ends_sequence(p, cur.nb, Hkv)) {
          cur.P += cur.nb;
          do {
            ++cur.b;
            if (cur.b >= B) return fail("walk ran past the batch", cs, w, cur.b, -1);
            cur.nb = nt[cur.b];
          } while (cur.nb == 0);
        }
      }
      if (taken != R1 - R0) return fail("workgroup took a different tile count", cs, w, -1, -1);
    }
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < Hkv; ++g) {
        if (nt[b] == 0) continue;
        for (int t = 0; t < nt[b]; ++t)
          if (cov[b][g][t] != 1) return fail("tile not taken exactly once", cs, -1, b, g);
        const int pieces = (int)seen_slots[b][g].size();
        if (recorded[b][g] != pieces) return fail("recorded piece count differs", cs, -1, b, g);
        std::vector<int> hit(slots, 0);
        for (int s : seen_slots[b][g]) hit[s]++;
        for (int s = 0; s < pieces; ++s)
          if (hit[s] != 1) return fail("slots are not 0..pieces-1", cs, -1, b, g);
        if ((pieces == 1) != (direct_seen[b][g] == 1))
          return fail("direct flag does not match one piece", cs, -1, b, g);
      }
  }
  std::printf("OK cases=%d pieces=%lld\n", cases, total_pieces);
  return 0;
}
