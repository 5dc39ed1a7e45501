// Integer arithmetic of the even-work grid, shared by the kernels (which
// call it from every workgroup) and by a host-compiled replay that checks the
// partition on the CPU.  Plain integer code with no device intrinsics.
//
// The decode tiles of all (sequence, kv head) units are laid end to end,
// units ordered by sequence then kv head, a unit of sequence b being n_b
// 16-key tiles: N = Hkv * sum_b n_b tiles.  Workgroup w of nw takes tiles
// [w*Wt, min((w+1)*Wt, N)), Wt = max(ceil(N / nw), min_tiles).  A unit of
// n_b <= max_tiles tiles with min_tiles = ceil(max_tiles / S) spans at most
// S + 1 workgroups, one partial slot each (slot = workgroup - first
// workgroup of the unit); the workgroup holding the unit's last tile records
// the unit's piece count.
#pragma once

#ifdef __HIPCC__
#define PA_HOST_DEVICE __host__ __device__
#else
#define PA_HOST_DEVICE
#endif

namespace pa {
namespace even_plan {

// Tiles per workgroup for N tiles over nw workgroups (nw >= 1).
PA_HOST_DEVICE inline long long tiles_per_workgroup(long long N, int nw, long long min_tiles) {
  const long long fill = (N + nw - 1) / nw;
  return fill > min_tiles ? fill : min_tiles;
}

// One piece of a workgroup's range: tiles [t0, t1) of unit (b, g), written to
// partial slot `slot` unless the unit fits in one workgroup (`direct`); the
// unit is cut into `pieces` pieces, and `last` marks the workgroup that holds
// its final tile (it records `pieces`).
struct Piece {
  int g, t0, t1, slot, pieces;
  bool direct, last;
};

// Cursor of a workgroup's walk: it is at tile `pos` (< R1) of the global
// order, inside sequence b, whose units start at global tile P * Hkv and have
// nb tiles each.
struct Cursor {
  long long pos, P;
  int b, nb;
};

// The piece at the cursor, for workgroup w with ranges of Wt tiles ending
// at R1.
PA_HOST_DEVICE inline Piece piece_at(const Cursor& c, long long R1, long long Wt, int Hkv, int w) {
  Piece p;
  const long long rel = c.pos - c.P * Hkv;
  p.g = (int)(rel / c.nb);
  p.t0 = (int)(rel % c.nb);
  const long long left = R1 - c.pos;
  const long long take = (long long)(c.nb - p.t0) < left ? (long long)(c.nb - p.t0) : left;
  p.t1 = p.t0 + (int)take;
  const long long u0 = c.P * Hkv + (long long)p.g * c.nb;  // first tile of the unit
  const int w_first = (int)(u0 / Wt);
  const int w_last = (int)((u0 + c.nb - 1) / Wt);
  p.pieces = w_last - w_first + 1;
  p.slot = w - w_first;
  p.direct = p.pieces == 1;
  p.last = w == w_last;
  return p;
}

// Whether the walk moves to the next sequence after piece p (the piece ended
// the last kv head's unit of this sequence).
PA_HOST_DEVICE inline bool ends_sequence(const Piece& p, int nb, int Hkv) {
  return p.g == Hkv - 1 && p.t1 == nb;
}

}  // namespace even_plan
}  // namespace pa
