// Paged GQA decode body (split-KV), for gfx950.
//
// One workgroup = (split, kv head, sequence); its W wavefronts stream the
// split's 16-key tiles round-robin (with pages of P = 16 * 2^s slots, tile t
// is slots 16 * (t mod 2^s) .. + 15 of block-table entry t >> s), each with
// its own online-softmax state, and merge through LDS at the end.
//
// Per tile and wavefront:
//   * K is read straight from HBM into the A operand of one
//     v_mfma_f32_16x16x32_bf16 per 32 dims (lane l reads 16 bytes of the K
//     row of key sigma(l % 16)); the query heads of this KV head form the B
//     operand, repeated across the 16 columns when G < 16 (the Q-Block step
//     of the IBM Triton summary's five-step list: K and V are read once for
//     all G heads).  S^T lands so that lane (c, n) holds head n % G for keys
//     c, c+4, c+8, c+12 of the tile.
//   * Online softmax in the log2 domain (scale*log2(e) folded into one
//     multiply); the running maximum is raised lazily, only when a tile's
//     maximum exceeds it by more than 8, so exponentials stay below 2^8 and
//     the accumulator is rescaled rarely (the m / l recurrence of the guide's
//     "Flash Attention革命" section).
//   * P.V in fp32 on the VALU: lane (c, n) owns dims 8n..8n+7 of keys
//     c + 4i; V rows are 16-byte coalesced loads (four full 256-byte rows per
//     instruction).  P stays fp32, so no rounding is added to the weights.
//   * Each wavefront keeps a ring of DEPTH tiles: the loads of the next
//     DEPTH - 1 tiles are in flight while one tile is computed.
// Masked keys (past the context, or stale NaN slots of the last page) are
// removed by select, never by arithmetic.
//
// Split-KV (the parallel tiled softmax step of the same list): a sequence
// with n_act > 1 non-empty splits writes normalised partials (O_k, lse_k) to
// the workspace, merged by log-sum-exp either in a second launch
// (splitkv_reduce_kernel / unit_merge_kernel, the default) or, with FUSED,
// by the last of its workgroups to finish (an agent-scope atomic counter per
// (sequence, kv head), released and acquired with device fences, reset to
// zero by the merging workgroup).  On gfx950 each agent-scope release writes
// back the XCD's L2, which costs more than the second launch.  A sequence
// with one non-empty split writes its output directly.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace decode_detail {

constexpr float kLazyThreshold = 8.0f;

template <int G>
__device__ __forceinline__ float head_bcast(float v, int h, int lane) {
  if constexpr (G == 1) {
    return v;
  } else if constexpr (G <= 4) {
    switch (h) {
      case 0: return quad_bcast<0>(v);
      case 1: return quad_bcast<1>(v);
      case 2: return quad_bcast<2>(v);
      default: return quad_bcast<3>(v);
    }
  } else {
    return shfl(v, (lane & 0x30) | h);
  }
}

__device__ __forceinline__ int readlane(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

// LDS floats decode_body needs from its caller: the wave merge takes
// W*G*D floats; the split merge takes G*kMaxSplits weights plus a
// [groups][G*D] reduction buffer (groups*G*D = max(G*D, 256W)).
template <int G, int W>
constexpr int decode_smem_floats() {
  constexpr int D = kHeadDim;
  constexpr int merge = G * kMaxSplits + (G * D > 256 * W ? G * D : 256 * W);
  return W * G * D > merge ? W * G * D : merge;
}

// The B operand: the G query heads of KV head g for query row qi (column n
// takes head n % G), 16 bytes of each of the four 32-dim k-steps per lane.
template <int G>
__device__ __forceinline__ void load_q_block(const DecodeParams& p, int qi, int g, int hl, int c,
                                             bf16x8 (&qb)[4]) {
  const uint16_t* qrow = p.q + ((int64_t)qi * p.num_q_heads + g * G + hl) * kHeadDim;
#pragma unroll
  for (int j = 0; j < 4; ++j) qb[j] = as_bf16x8(ld16(qrow + 32 * j + 8 * c));
}

// Lane byte offsets inside a (page, kv head) slice: K chunk of MFMA row n
// (key sigma(n), dims 8c..), V row chunk (key c, dims 8n..).  Below 2^31: a
// page spans fewer than 2^31 elements.
__device__ __forceinline__ uint32_t k_lane_offset(const DecodeParams& p, int c, int n) {
  const int ktok = (n >> 2) + 4 * (n & 3);  // sigma: MFMA row -> key in tile
  return (uint32_t)(2 * (ktok * (int)p.stride_token + 8 * c));
}
__device__ __forceinline__ uint32_t v_lane_offset(const DecodeParams& p, int c, int n) {
  return (uint32_t)(2 * (c * (int)p.stride_token + 8 * n));
}

// K and V of 16-key tile t of KV head g, whose block-table entry names
// `page`, into one ring slot: four 16-byte K chunks (the MFMA A operand)
// and four V rows of 16 bytes per lane.  The tile's base address is uniform
// (page, head and slot are the same on every lane), the lane offsets koff /
// voff are 32-bit, so each load is a scalar base plus a vector offset.
__device__ __forceinline__ void load_kv_tile(const DecodeParams& p, int g, int64_t page, int t,
                                             int pmask, int tok16, uint32_t koff, uint32_t voff,
                                             uint4 (&kr)[4], uint4 (&vr)[4]) {
  const int64_t off = page * p.stride_page + (int64_t)g * p.stride_head +
                      (int64_t)((t & pmask) * tok16);
  const char* kb = reinterpret_cast<const char*>(p.k_pool + off);
  const char* vb = reinterpret_cast<const char*>(p.v_pool + off);
  const int64_t vrow = 8 * p.stride_token;  // bytes between V rows 4 keys apart
#pragma unroll
  for (int j = 0; j < 4; ++j) kr[j] = *reinterpret_cast<const uint4*>(kb + koff + 64 * j);
#pragma unroll
  for (int r = 0; r < 4; ++r) vr[r] = *reinterpret_cast<const uint4*>((vb + r * vrow) + voff);
}

// One tile of one wavefront: the scores of keys 16t.. (those at or past L
// masked), the online-softmax update of (m, lsum, acc), and P.V.
template <int G>
__device__ __forceinline__ void tile_update(const DecodeParams& p, const uint4 (&kc)[4],
                                            uint4 (&vc)[4], const bf16x8 (&qb)[4], int t, int L,
                                            int c, int lane, float& m, float& lsum,
                                            float (&acc)[G][8]) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[j]), qb[j], s, 0, 0, 0);

  const int key0 = t * kDecodeTile + c;
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = (key0 + 4 * r < L) ? s[r] * p.scale_log2 : kNegInf;
  float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  tmax = fmaxf(tmax, shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, shfl_xor(tmax, 32));

  const bool need = tmax > m + kLazyThreshold;
  if (wave_any(need)) {
    const float m_new = need ? tmax : m;
    const float alpha = fast_exp2(m - m_new);  // 0 on the first tile
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ah = head_bcast<G>(alpha, h, lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= ah;
    }
  }

  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(x[r] - m);
  lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);

  if (t * kDecodeTile + kDecodeTile > L) {  // last tile: drop stale V rows
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (key0 + 4 * r >= L) vc[r] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v[8];
    v[0] = bf16lo(vc[r].x); v[1] = bf16hi(vc[r].x);
    v[2] = bf16lo(vc[r].y); v[3] = bf16hi(vc[r].y);
    v[4] = bf16lo(vc[r].z); v[5] = bf16hi(vc[r].z);
    v[6] = bf16lo(vc[r].w); v[7] = bf16hi(vc[r].w);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ph = head_bcast<G>(pr[r], h, lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, v[e], acc[h][e]);
    }
  }
}

// End of one (sequence, kv head) unit or piece of it: sum each wavefront's
// state over its four key groups, merge the W wavefronts through LDS and
// write the G rows, to the output (direct) or as normalised partials with
// their lse to slot `slot` of S (partial rows are per sequence, b * Hq + h).
// Ends with the LDS buffer still in use: callers that reuse it synchronise.
template <int G, int W>
__device__ __forceinline__ void merge_waves_and_store(const DecodeParams& p, float (&acc)[G][8],
                                                      float m, float lsum, int b, int g, int qi,
                                                      bool direct, int S, int slot,
                                                      float* sm_buf) {
  constexpr int D = kHeadDim;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane >> 4, n = lane & 15;
  // Sum this wavefront's partials over the four key groups.
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[h][e] += shfl_xor(acc[h][e], 16);
      acc[h][e] += shfl_xor(acc[h][e], 32);
    }

  // Merge the W wavefronts through LDS.
  __shared__ float sm_m[W][G];
  __shared__ float sm_l[W][G];
  if (c == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(&sm_buf[(wave * G + h) * D + 8 * n]);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
    if (n < G) {
      sm_m[wave][n] = m;
      sm_l[wave][n] = lsum;
    }
  }
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += 64 * W) {
    const int h = idx / D;
    const int d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][h]);
    float o = 0.f, l = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = sm_m[w][h];
        if (mw != kNegInf) {
          const float e = fast_exp2(mw - M);
          o = fmaf(e, sm_buf[(w * G + h) * D + d], o);
          l = fmaf(e, sm_l[w][h], l);
        }
      }
      o = o / l;
    }
    const float lse_nat = (M == kNegInf) ? kNegInf : (M + fast_log2(l)) * kLn2;
    const int64_t row = (int64_t)b * p.num_q_heads + g * G + h;  // partials: per sequence
    if (direct) {
      const int64_t orow = (int64_t)qi * p.num_q_heads + g * G + h;
      if (p.out_f32)
        reinterpret_cast<float*>(p.out)[orow * D + d] = o;
      else
        reinterpret_cast<uint16_t*>(p.out)[orow * D + d] = f2bf(o);
      if (p.lse && d == 0) p.lse[orow] = lse_nat;
    } else {
      p.part_o[(row * S + slot) * D + d] = o;
      if (d == 0) p.part_lse[row * S + slot] = lse_nat;
    }
  }
}

// Where a piece of one (sequence, kv head) unit goes in the even-work grid:
// tiles [t_begin, t_end), written straight to the output when the piece is
// the whole unit, else to partial slot `slot` of `slots`.
struct EvenPiece {
  int t_begin, t_end, slot, slots;
  bool direct;
};

// One workgroup of W wavefronts: split `split` of KV head g of sequence b
// (static grid), or, with EVEN, the piece `ev` of that unit.
// sm_buf: decode_smem_floats<G, W>() floats of LDS, 16-byte aligned.
template <int G, int W, bool FUSED, bool EVEN = false>
__device__ __forceinline__ void decode_body(const DecodeParams& p, int split, int g, int b,
                                            float* sm_buf, EvenPiece ev = EvenPiece{}) {
  static_assert(!(FUSED && EVEN), "the even-work grid merges in a separate kernel");
  constexpr int DEPTH = G <= 4 ? 3 : 2;  // tiles per wavefront ring (in flight + computing)
  constexpr int D = kHeadDim;
  static_assert(G * W <= 128, "LDS budget: W x G x D floats (64 KiB at G = 16, W = 8)");
  const int tid = threadIdx.x;
  // Query / output row of sequence b: b itself, or its single query token
  // inside a mixed batch (sequences with more query tokens are not decode
  // rows and exit).
  int qi = b;
  if (p.query_start_loc) {
    qi = p.query_start_loc[b];
    if (p.query_start_loc[b + 1] - qi != 1) return;
  }
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane >> 4;  // key group: keys c + 4i of a tile
  const int n = lane & 15;  // MFMA column; head n % G; dims 8n..8n+7 in P.V
  const int hl = n % G;

  // Loads that do not depend on the context length go first, so they overlap
  // its load: this KV head's query heads (B operand, column n -> head n % G)
  // and the page ids of this wave's first 64 tiles (lane i: tile
  // split*tps + wave + W*i, read only inside the block-table row).
  const int tps = p.tiles_per_split;
  const int t_begin = EVEN ? ev.t_begin : split * tps;
  bf16x8 qb[4];
  load_q_block<G>(p, qi, g, hl, c, qb);
  // 16-key tile t lies in block-table entry t >> page_shift, 16 * (t & pmask)
  // slots into that page
  const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks;
  const int ps = p.page_shift, pmask = (1 << p.page_shift) - 1;
  const int tok16 = 16 * (int)p.stride_token;  // < 2^31: a page spans < 2^31 elements
  const int t_first = t_begin + wave + W * lane;
  int pages = ((t_first >> ps) < p.max_blocks) ? bt[t_first >> ps] : 0;

  const int L = p.context_lens[b];
  // A context beyond the host bound is undefined behaviour; clamping here only
  // keeps every access inside the block table and the workspace.
  const int ntiles = EVEN ? ev.t_end
                        : min((L + kDecodeTile - 1) / kDecodeTile,
                              min(p.max_blocks << ps, p.num_splits * tps));
  const int n_act = EVEN ? 1 : (ntiles + tps - 1) / tps;  // non-empty splits of this sequence
  if (!EVEN && split >= (n_act > 1 ? n_act : 1)) {
    // Unfused merge: the separate reduce reads every split, so an empty one
    // marks its rows with lse = -inf (weight 0).
    if (!FUSED && tid < G)
      p.part_lse[((int64_t)b * p.num_q_heads + g * G + tid) * p.num_splits + split] = kNegInf;
    return;
  }
  const int t_end = EVEN ? ev.t_end : min(t_begin + tps, ntiles);
  // tiles of this wavefront: t_begin + wave + W*i, i < nt
  const int nt = (t_end - t_begin - wave + W - 1) / W > 0 ? (t_end - t_begin - wave + W - 1) / W : 0;

  const uint32_t koff = k_lane_offset(p, c, n), voff = v_lane_offset(p, c, n);

  // Page ids of later chunks, 64 tiles at a time: lane i holds the page of
  // this wave's tile chunk*64 + i.
  auto fetch_pages = [&](int chunk) {
    const int i = lane + 64 * chunk;
    pages = (i < nt) ? bt[(t_begin + wave + W * i) >> ps] : 0;
  };
  int chunk_base = 0;  // first tile index (of this wave's list) of the current chunk
  auto issue = [&](int i, uint4 (&kr)[4], uint4 (&vr)[4]) {
    load_kv_tile(p, g, readlane(pages, i & 63), t_begin + wave + W * (chunk_base + i), pmask,
                 tok16, koff, voff, kr, vr);
  };

  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m = kNegInf;  // running log2-domain max for head hl
  float lsum = 0.f;   // partial softmax denominator (this lane's keys)

  uint4 kr[DEPTH][4], vr[DEPTH][4];

  auto process = [&](uint4 (&kc)[4], uint4 (&vc)[4], int i) {
    tile_update<G>(p, kc, vc, qb, t_begin + wave + W * i, L, c, lane, m, lsum, acc);
  };

  // Software pipeline over chunks of 64 tiles.  Tile i of a chunk lives in
  // ring slot i % DEPTH; the loads of the next DEPTH - 1 tiles are in flight
  // while one tile is computed.  No load sits under a branch inside the
  // pipelined loop (past the chunk end the index is clamped to its last
  // tile, an L2 hit), so the compiler can wait on exact load counts instead
  // of draining every outstanding load.
  for (int cb = 0; cb < nt; cb += 64) {
    const int n = min(64, nt - cb);
    chunk_base = cb;
    if (cb > 0) fetch_pages(cb >> 6);
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) issue(min(d, n - 1), kr[d], vr[d]);
    int i0 = 0;
    for (; i0 + DEPTH <= n; i0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        constexpr int kAhead = DEPTH - 1;
        issue(min(i0 + d + kAhead, n - 1), kr[(d + kAhead) % DEPTH], vr[(d + kAhead) % DEPTH]);
        process(kr[d], vr[d], cb + i0 + d);
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
      if (i0 + d < n) process(kr[d], vr[d], cb + i0 + d);
  }

  __shared__ float sm_head[2][G];
  __shared__ int sm_last;
  const int S = EVEN ? ev.slots : p.num_splits;
  const int slot = EVEN ? ev.slot : split;
  const bool direct = EVEN ? ev.direct : (FUSED ? n_act <= 1 : S == 1);
  merge_waves_and_store<G, W>(p, acc, m, lsum, b, g, qi, direct, S, slot, sm_buf);
  if (direct || !FUSED) return;

  // Split-KV: count this split in; the last one merges.  The barrier makes
  // every wave's partial stores complete; thread 0's agent-scope release RMW
  // then publishes them (one L2 write-back per workgroup), and only the
  // merging workgroup pays for an acquire (L2 invalidate).
  __syncthreads();
  if (tid == 0) {
    int* ctr = p.counters + (int64_t)b * p.num_kv_heads + g;
    const int prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    sm_last = (prev == n_act - 1);
    if (sm_last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!sm_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // Merge weights: w[h][k] = exp(lse_k - M_h) for the n_act splits.
  float* wts = sm_buf;  // [G][n_act], reuses the wave-merge buffer
  const int64_t row0 = (int64_t)b * p.num_q_heads + g * G;
  for (int idx = tid; idx < G * n_act; idx += 64 * W) {
    const int h = idx / n_act, k = idx % n_act;
    wts[h * n_act + k] = p.part_lse[(row0 + h) * S + k];
  }
  __syncthreads();
  if (wave == 0) {
    for (int h = 0; h < G; ++h) {
      float M = kNegInf;
      for (int k = lane; k < n_act; k += 64) M = fmaxf(M, wts[h * n_act + k]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
      float sum = 0.f;
      for (int k = lane; k < n_act; k += 64) sum += fast_exp2((wts[h * n_act + k] - M) * kLog2e);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += shfl_xor(sum, off);
      if (lane == 0) {
        sm_head[0][h] = M;
        sm_head[1][h] = sum;
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * n_act; idx += 64 * W) {
    const int h = idx / n_act;
    wts[idx] = fast_exp2((wts[idx] - sm_head[0][h]) * kLog2e) / sm_head[1][h];
  }
  __syncthreads();

  // O = sum_k w_k O_k: work item (group, head, 4 dims), k strided over the
  // groups; every thread takes items tid, tid + 64W, ...
  constexpr int kItems = G * D / 4;
  constexpr int kGroups = (64 * W) / kItems > 0 ? (64 * W) / kItems : 1;
  float* red = sm_buf + G * kMaxSplits;  // [kGroups][G*D]
  for (int it = tid; it < kItems * kGroups; it += 64 * W) {
    const int item = it % kItems;
    const int grp = it / kItems;
    const int h = item / (D / 4);
    const int d0 = (item % (D / 4)) * 4;
    const float* src = p.part_o + (row0 + h) * S * D + d0;
    float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
    int k = grp;
    for (; k + 7 * kGroups < n_act; k += 8 * kGroups) {  // eight loads in flight
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const float4*>(src + (int64_t)(k + u * kGroups) * D);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = wts[h * n_act + k + u * kGroups];
        o4.x = fmaf(w, v[u].x, o4.x);
        o4.y = fmaf(w, v[u].y, o4.y);
        o4.z = fmaf(w, v[u].z, o4.z);
        o4.w = fmaf(w, v[u].w, o4.w);
      }
    }
    for (; k < n_act; k += kGroups) {
      const float w = wts[h * n_act + k];
      const float4 ok = *reinterpret_cast<const float4*>(src + (int64_t)k * D);
      o4.x = fmaf(w, ok.x, o4.x);
      o4.y = fmaf(w, ok.y, o4.y);
      o4.z = fmaf(w, ok.z, o4.z);
      o4.w = fmaf(w, ok.w, o4.w);
    }
    *reinterpret_cast<float4*>(&red[grp * G * D + 4 * item]) = o4;
  }
  __syncthreads();
  for (int idx = tid; idx < kItems; idx += 64 * W) {
    float4 acc4 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q = 0; q < kGroups; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(&red[q * G * D + 4 * idx]);
      acc4.x += v.x; acc4.y += v.y; acc4.z += v.z; acc4.w += v.w;
    }
    const int h = idx / (D / 4);
    const int d0 = (idx % (D / 4)) * 4;
    const int64_t row = (int64_t)qi * p.num_q_heads + g * G + h;
    if (p.out_f32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row * D + d0) = acc4;
    } else {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * D + d0) =
          make_uint2(pack_bf16x2(acc4.x, acc4.y), pack_bf16x2(acc4.z, acc4.w));
    }
    if (p.lse && d0 == 0) p.lse[row] = sm_head[0][h] + fast_log2(sm_head[1][h]) * kLn2;
  }
}

}  // namespace decode_detail
}  // namespace pa
