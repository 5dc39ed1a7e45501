// Paged GQA prefill body (bf16 MFMA) for gfx950.
//
// One workgroup = (query tile of one sequence, kv head).  Its Q-block is
// 256 rows (128 at head dim 256): QT = rows / G query tokens x the G query
// heads that share the KV head (the Q-Block step of the IBM Triton summary's
// five-step list), row r -> token r / G, head r % G; wavefront w owns rows
// 32w..32w+31 and each lane owns one row (lane % 32).  The workgroup walks
// the sequence's keys in tiles of 32 (two 16-slot blocks of its pages), up
// to the causal limit of its last token, staging each K and V tile in LDS
// once for all its wavefronts (FlashAttention-style
// tiling, guide sections "Flash Attention革命" and "Triton实现Flash
// Attention"):
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, K rows from LDS (16-byte reads),
//                 Q^T held in registers; lane l receives 16 keys of row l%32.
//   online softmax in the log2 domain with a lazily raised running max;
//   masked keys (past the context, or after the row's causal position) are
//   removed by select.
//   O^T += V^T P^T  v_mfma_f32_32x32x16_bf16; P (rounded to bf16) is already
//                 in the B-operand layout the S^T result left it in; V stays
//                 row-major in LDS and V^T comes out of ds_read_b64_tr_b16
//                 (each 16-lane group transposes a 4-key x 16-dim block).
//                 The precise variant splits P into a bf16 high part and a
//                 bf16 remainder (two MFMAs), leaving a relative weight error
//                 of about 2^-18 instead of 2^-9.
// Each sequence's query tokens are the last q_len positions of its context:
// query token i sees keys j <= L - q_len + i (bottom-right causal alignment,
// so a chunk attends to its cached prefix in full).  The grid is static:
// x runs over a host bound on query tiles; each workgroup finds its
// sequence by a scan of query_start_loc and surplus workgroups exit.
// With tile_splits = S > 1 the tile's key tiles are dealt out in S
// contiguous runs (the parallel tiled softmax of the five-step list applied
// to a query tile), each run writes normalised partials and their lse, and
// tile_merge_kernel combines them by log-sum-exp.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace prefill_detail {

constexpr int kWaves = 8;            // wavefronts per workgroup at head dims 64 and 128
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;   // Q-block rows per workgroup
constexpr int kKvTile = 32;          // keys per inner step
// Head dim 256 holds 128 output accumulators per lane for its 32 rows, so
// its workgroup is four wavefronts, one per SIMD with the whole register
// file, and its Q-block 128 rows.
template <int D>
constexpr int waves_of() {
  return D == 256 ? 4 : kWaves;
}
template <int D>
constexpr int rows_of() {
  return 32 * waves_of<D>();
}
// K and V LDS rows (bf16 elements) for head dim D: K rows padded by 8
// (272 B at D = 128: the 16-byte row reads of sixteen lanes cover all 64
// banks once); V rows padded by 32 (320 B at 128, 192 B at 64: consecutive
// rows start 16 banks apart, so the four rows a transposing read group
// touches, and the four more of the other group of the same 32 lanes, fall
// on disjoint banks); at 256, V rows are padded by 16 (544 B: rows 8 banks
// apart, disjoint over a group's four rows) so that the ring fits in LDS.
template <int D>
constexpr int k_stride() {
  return D + 8;
}
template <int D>
constexpr int v_stride() {
  return D == 256 ? D + 16 : D + 32;
}
constexpr int kKBufs = 4;                 // LDS K tile buffers
constexpr int kVBufs = 5;                 // LDS V tile buffers (V is read one step later)
// 16-key blocks of the LDS page window (one 64-bit byte offset each): 2048
// (32k keys), 1024 (16k keys) at head dim 256
template <int D>
constexpr int page_cache() {
  return D == 256 ? 1024 : 2048;
}
constexpr float kLazyThreshold = 8.0f;

// Find (sequence, query tile) of workgroup x: tiles are numbered sequence by
// sequence, ceil(q_len / qt) per sequence (none for single-token sequences
// when skip_single: those run as decode workgroups).  Returns false for a
// surplus x.  W: wavefronts of the calling workgroup.
template <int W = kWaves>
__device__ bool find_tile(const int32_t* qsl, int num_seqs, int qt, int x, bool skip_single,
                          int* seq, int* tile) {
  __shared__ int s_found[2];
  __shared__ int s_wsum[W];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_found[0] = -1;
  int base = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += 64 * W) {
    const int s = c0 + tid;
    int cnt = 0;
    if (s < num_seqs) {
      const int ql = qsl[s + 1] - qsl[s];
      cnt = (skip_single && ql == 1) ? 0 : (ql + qt - 1) / qt;
    }
    int v = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    __syncthreads();
    if (lane == 63) s_wsum[wave] = v;
    __syncthreads();
    int wbase = 0, total = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      if (w < wave) wbase += s_wsum[w];
      total += s_wsum[w];
    }
    const int incl = base + wbase + v;
    if (cnt > 0 && x >= incl - cnt && x < incl) {
      s_found[0] = s;
      s_found[1] = x - (incl - cnt);
    }
    base += total;
    __syncthreads();
    if (s_found[0] >= 0 || x < base) break;
  }
  *seq = s_found[0];
  *tile = s_found[1];
  return s_found[0] >= 0;
}

// LDS bytes prefill_body needs from its caller (K tiles, V^T tiles, the
// page window's block offsets).
template <int D = kHeadDim>
constexpr int prefill_smem_bytes() {
  return kKBufs * kKvTile * k_stride<D>() * 2 + kVBufs * kKvTile * v_stride<D>() * 2 +
         page_cache<D>() * 8;
}

// One workgroup of 64 * waves_of<D>() threads: query tile / split / KV head
// number `id` of the 1-D prefill grid (nx tiles x tile_splits x Hkv), head
// dim D (64, 128 or 256).  smem: prefill_smem_bytes<D>(), 16-byte aligned.
template <int G, bool PRECISE, int D = kHeadDim>
__device__ __forceinline__ void prefill_body(const PrefillParams& p, int id, int nx,
                                             char* smem) {
  static_assert(D == 64 || D == 128 || D == 256, "query tiles are built for 64, 128 and 256");
  constexpr int W = waves_of<D>();
  constexpr int T = 64 * W;   // threads
  constexpr int kLdsStride = k_stride<D>();
  constexpr int kVStride = v_stride<D>();
  constexpr int KS = D / 16;  // k-steps of the S^T MFMA
  constexpr int MT = D / 32;  // 32-dim M tiles of O^T
  constexpr int QT = rows_of<D>() / G;
  // 1-D grid: id -> (kv head, split, query tile).  Consecutive ids go to
  // different XCDs, so with Hkv = 8 each XCD serves one KV head and its K/V
  // stay in that XCD's L2.  Query tiles run from the last (heaviest under the
  // causal mask) to the first.
  const int g = id % p.num_kv_heads;
  const int nsplit = p.tile_splits;
  const int split = (id / p.num_kv_heads) % nsplit;
  const int x = nx - 1 - id / (p.num_kv_heads * nsplit);
  int s, qtile;
  if (!find_tile<W>(p.query_start_loc, p.num_seqs, QT, x, p.decode_rows_apart != 0, &s, &qtile))
    return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, half = lane >> 5;
  const int q0 = p.query_start_loc[s];
  const int qlen = p.query_start_loc[s + 1] - q0;
  const int L = p.context_lens[s];
  const int tok0 = qtile * QT;
  const int ntok = min(QT, qlen - tok0);

  // This lane's row: token r / G, head r % G.
  const int r = 32 * wave + n;  // < 32 W
  const int tl = r / G, h = r % G;
  const bool row_valid = tl < ntok;
  const int qi = tok0 + tl;  // index of the token inside the chunk
  const int key_limit = p.causal ? min(L, L - qlen + qi + 1) : L;  // keys < limit
  // smallest limit among this wave's rows (its first token): tiles that end
  // below it need no mask
  const int wave_limit = p.causal ? min(L, L - qlen + tok0 + (32 * wave) / G + 1) : L;
  const int kv_end = p.causal ? min(L, L - qlen + tok0 + ntok) : L;
  const int nkv_all = kv_end > 0 ? (kv_end + kKvTile - 1) / kKvTile : 0;
  // this workgroup's run of key tiles [j0, j0 + nkv)
  const int per = nsplit > 1 ? (nkv_all + nsplit - 1) / nsplit : nkv_all;
  const int j0 = min(nkv_all, split * per);
  const int nkv = min(nkv_all - j0, per);
  const int64_t orow = (int64_t)(q0 + qi) * p.num_q_heads + g * G + h;
  if (nsplit > 1 && nkv <= 0) {  // empty run: weight zero in the merge
    if (row_valid && half == 0) p.tpart_lse[orow * nsplit + split] = kNegInf;
    return;
  }

  // Q^T operand: lane holds Q[row][16ks + 8*half .. +8] for ks < KS.
  bf16x8 qb[KS];
  {
    const uint16_t* qrow = p.q + ((int64_t)(q0 + qi) * p.num_q_heads + g * G + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = row_valid ? as_bf16x8(ld16(qrow + 16 * ks)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  // LDS: kKBufs K tiles and kVBufs V tiles, both row-major [key][dim]
  // (padded rows); the step loop below says which tile each buffer holds
  // when.
  auto k_lds = reinterpret_cast<uint16_t(*)[kKvTile * kLdsStride]>(smem);
  auto v_lds =
      reinterpret_cast<uint16_t(*)[kKvTile * kVStride]>(smem + kKBufs * kKvTile * kLdsStride * 2);

  // Tile loader.  D = 128: thread t stages 16 bytes of K and 16 bytes of V
  // of key t / 16, dims 8*(t%16) .. +7 (a wavefront moves four whole
  // 256-byte rows of each), so every wavefront does the same staging work.
  // D = 64: a tile is 256 chunks of 16 bytes for K and as many for V, so
  // wavefronts 0..3 stage K and 4..7 stage V.  D = 256 (256 threads): a tile
  // is 1024 chunks of each, so thread t stages chunk t % 32 of keys
  // t / 32 + 8i, i = 0..3 (keys 0..15 of the tile's first page, 16..31 of
  // its second).  Loads are unconditional (a key past the context reads a
  // valid page and its V row is zeroed when stored), so no load sits under a
  // branch and the compiler keeps them in flight across the loop.
  constexpr int CH = D / 8;  // 16-byte chunks per row
  constexpr bool kSplitKV = 2 * kKvTile * CH <= T;
  constexpr int NC = kSplitKV ? 1 : kKvTile * CH / T;  // chunks of K (and of V) per thread
  constexpr int KSTEP = T / CH;                          // key step between a thread's chunks
  static_assert(kSplitKV || NC * T == kKvTile * CH, "whole chunks per thread");
  static_assert(NC == 1 || (KSTEP * 2 == kPage && NC == 4), "multi-chunk staging: D = 256");
  const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks;
  const int ti = kSplitKV ? tid % (kKvTile * CH) : tid;
  const bool stage_v = kSplitKV && tid >= kKvTile * CH;  // wavefront-uniform
  const int lkey = ti / CH, ldc = ti % CH;
  const int64_t loff = (int64_t)g * p.stride_head + (int64_t)(lkey % kPage) * p.stride_token + 8 * ldc;
  const char* kth = reinterpret_cast<const char*>(p.k_pool + loff);
  const char* vth = reinterpret_cast<const char*>(p.v_pool + loff);
  // multi-chunk staging: the odd chunks sit KSTEP slots further into a page
  const uint32_t odd_bytes = (uint32_t)(KSTEP * p.stride_token * 2);
  const uint32_t page_bytes = (uint32_t)(p.stride_page * 2);  // < 2^32 (checked on the host)
  // Byte offsets of the 16-key blocks of the current window of key tiles
  // (block j: page bt[j >> page_shift], slots 16 * (j & pmask) ..), staged in
  // LDS, keep the block-table lookup and the address arithmetic off each
  // tile's load path.  Blocks past the context hold offset 0 (page 0, never
  // used: those keys are masked and zeroed).
  uint64_t* pg_lds = reinterpret_cast<uint64_t*>(smem + kKBufs * kKvTile * kLdsStride * 2 +
                                                 kVBufs * kKvTile * kVStride * 2);
  constexpr int kWinTiles = page_cache<D>() * kPage / kKvTile;
  const int ps = p.page_shift, pmask = (1 << p.page_shift) - 1;
  const uint32_t block_bytes = (uint32_t)(kPage * p.stride_token * 2);  // 16 slots of a page
  // valid 16-key blocks: inside the context and the block table
  const int nblk = min((L + kPage - 1) / kPage, p.max_blocks << ps);
  int win0 = 0;                              // first key tile of the window
  // tile t of the window -> r[i] = K chunk i, r[NC + i] = V chunk i (split:
  // r[0] = this thread's K or V chunk)
  constexpr int NR = kSplitKV ? 1 : 2 * NC;
  auto load_tile = [&](int t, uint4 (&r)[NR]) {
    if constexpr (kSplitKV) {
      const uint64_t off = pg_lds[t * (kKvTile / kPage) + lkey / kPage];
      r[0] = *reinterpret_cast<const uint4*>((stage_v ? vth : kth) + off);
    } else if constexpr (NC == 1) {
      const uint64_t off = pg_lds[t * (kKvTile / kPage) + lkey / kPage];
      r[0] = *reinterpret_cast<const uint4*>(kth + off);
      r[1] = *reinterpret_cast<const uint4*>(vth + off);
    } else {
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const uint64_t off = pg_lds[t * (kKvTile / kPage) + i / 2] + ((i & 1) ? odd_bytes : 0u);
        r[i] = *reinterpret_cast<const uint4*>(kth + off);
        r[NC + i] = *reinterpret_cast<const uint4*>(vth + off);
      }
    }
  };
  auto store_tile = [&](int t, int kbuf, int vbuf, const uint4 (&r)[NR]) {
    // V rows past the context are zeroed: stale data (even NaN) must not
    // reach O through a zero weight
    const bool tail = (win0 + t + 1) * kKvTile > L;  // uniform
    // element-wise copies: a whole-struct copy becomes a memcpy that can
    // keep the staging registers in memory
    if constexpr (kSplitKV || NC == 1) {
      const bool dead = tail && (win0 + t) * kKvTile + lkey >= L;
      const uint32_t keep = dead ? 0u : ~0u;
      if constexpr (kSplitKV) {
        if (stage_v)
          *reinterpret_cast<uint4*>(&v_lds[vbuf][lkey * kVStride + 8 * ldc]) =
              make_uint4(r[0].x & keep, r[0].y & keep, r[0].z & keep, r[0].w & keep);
        else
          *reinterpret_cast<uint4*>(&k_lds[kbuf][lkey * kLdsStride + 8 * ldc]) =
              make_uint4(r[0].x, r[0].y, r[0].z, r[0].w);
      } else {
        *reinterpret_cast<uint4*>(&k_lds[kbuf][lkey * kLdsStride + 8 * ldc]) =
            make_uint4(r[0].x, r[0].y, r[0].z, r[0].w);
        *reinterpret_cast<uint4*>(&v_lds[vbuf][lkey * kVStride + 8 * ldc]) =
            make_uint4(r[1].x & keep, r[1].y & keep, r[1].z & keep, r[1].w & keep);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int key = lkey + KSTEP * i;
        const bool dead = tail && (win0 + t) * kKvTile + key >= L;
        const uint32_t keep = dead ? 0u : ~0u;
        *reinterpret_cast<uint4*>(&k_lds[kbuf][key * kLdsStride + 8 * ldc]) =
            make_uint4(r[i].x, r[i].y, r[i].z, r[i].w);
        *reinterpret_cast<uint4*>(&v_lds[vbuf][key * kVStride + 8 * ldc]) =
            make_uint4(r[NC + i].x & keep, r[NC + i].y & keep, r[NC + i].z & keep,
                       r[NC + i].w & keep);
      }
    }
  };
  // Transposing V reads: lane (group gq = lane / 16, r = lane % 16) points
  // at key 4*half + r/4 (+16kk, +8 for the second read), dims
  // 16*(gq%2) + 4*(r%4) (+32mt); it receives dim 16*(gq%2) + r (+32mt) for
  // keys +0..3, the A-operand layout that matches P's B-operand keys
  // 16kk + 8*(j/4) + 4*half + j%4.
  const int vr_off = (4 * half + (lane & 15) / 4) * kVStride + 16 * ((lane >> 4) & 1) +
                     4 * (lane & 3);
  // S^T = K Q^T for the tile in buffer buf, D in KS steps of 16.  All K
  // operands are read before the first MFMA (the scheduling barrier
  // keeps the compiler from sinking each read next to its MFMA, which would
  // put an LDS round trip between every pair of dependent MFMAs).
  auto qk = [&](int buf, f32x16& st) {
    bf16x8 ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // two 8-byte LDS reads: measured faster than one 16-byte read on gfx950
      const uint16_t* kr = &k_lds[buf][n * kLdsStride + 16 * ks + 8 * half];
      const uint2 a0 = *reinterpret_cast<const uint2*>(kr);
      const uint2 a1 = *reinterpret_cast<const uint2*>(kr + 4);
      ka[ks] = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 16; ++e) st[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qb[ks], st, 0, 0, 0);
  };

  f32x16 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[mt][e] = 0.f;
  float m = kNegInf, lsum = 0.f;
  const float c = p.scale_log2;  // > 0 (checked on the host)
  f32x16 st_cur, st_next;

  // Softmax of key tile jg (its S^T in st_cur): P rounded to bf16 in pk
  // (and its bf16 remainder in pl for the precise variant), the running max
  // and sum updated, O rescaled when the max rises.
  uint32_t pk[8], pl[8];
  auto softmax = [&](int jg) {
    // Register e holds key 8*(e/4) + 4*half + e%4 of the tile, row n; the
    // log2-domain logit is c*S (c > 0, so the max can be taken on S).
    const bool full = jg * kKvTile + kKvTile <= wave_limit;  // no key of the tile masked
    if (!full) {
      const int kbase = jg * kKvTile + 4 * half;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + 8 * (e >> 2) + (e & 3);
        st_cur[e] = (key < key_limit) ? st_cur[e] : kNegInf;
      }
    }
    float smax = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; ++e) smax = fmaxf(smax, st_cur[e]);
    const f32x2 hm = halves(smax);
    const float tmax = fmaxf(hm[0], hm[1]) * c;
    const bool need = tmax > m + kLazyThreshold;
    if (wave_any(need)) {
      const float m_new = need ? tmax : m;
      const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[mt][e] *= alpha;
    }
    const float neg_m = (m == kNegInf) ? 0.f : -m;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = fast_exp2(fmaf(st_cur[e], c, neg_m));
      const float p1 = fast_exp2(fmaf(st_cur[e + 1], c, neg_m));
      pk[e >> 1] = pack_bf16x2(p0, p1);
      if constexpr (PRECISE) {
        psum += p0 + p1;
        pl[e >> 1] = pack_bf16x2(p0 - bf16lo(pk[e >> 1]), p1 - bf16hi(pk[e >> 1]));
      }
    }
    // (with P rounded to bf16, its row sum is taken in the MFMA phase that
    // multiplies P by V, beside that phase's MFMAs: see pv)
    if constexpr (PRECISE) lsum += psum;
  };

  // O^T += V^T P^T for the tile whose V is in buffer vbuf and whose P is in
  // pk / pl: two k-steps of 16 keys, four 32-dim M tiles.  The buffer's base
  // address is made opaque, so each of the sixteen reads is that base plus a
  // constant the instruction's offset field holds (left alone, the compiler
  // keeps sixteen hoisted addresses in registers and rebuilds each one every
  // tile).
  auto pv = [&](int vbuf) {
    if constexpr (!PRECISE) {
      // the row sum of the weights the MFMA uses (P rounded to bf16); it is
      // added here, before the next tile's softmax can rescale lsum, so that
      // its VALU work sits in the MFMA phase, where the SIMD has issue slots
      // to spare, instead of lengthening the softmax phase
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) psum = add_bf16x2(pk[e], psum);
      lsum += psum;
      asm volatile("" : "+v"(lsum));  // keep the sum in this phase
    }
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    lds_i16x4* vb = (lds_i16x4*)&v_lds[vbuf][vr_off];
    asm volatile("" : "+v"(vb));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pk[4 * kk], pk[4 * kk + 1],
                                                              pk[4 * kk + 2], pk[4 * kk + 3]));
      bf16x8 pbl;
      if constexpr (PRECISE)
        pbl = __builtin_bit_cast(bf16x8, make_uint4(pl[4 * kk], pl[4 * kk + 1], pl[4 * kk + 2],
                                                    pl[4 * kk + 3]));
      bf16x8 va[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // element offsets / 4: one i16x4 is 4 bf16
        lds_i16x4* at = vb + (16 * kk * kVStride + 32 * mt) / 4;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at + 8 * kVStride / 4);
        va[mt] = __builtin_bit_cast(
            bf16x8, make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                               __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[mt], pb, o[mt], 0, 0, 0);
        if constexpr (PRECISE)
          o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[mt], pbl, o[mt], 0, 0, 0);
      }
    }
  };

  // The run [j0, j0 + nkv) in windows of at most kWinTiles key tiles (one
  // LDS window of block offsets each).  Each step j is two phases, each ending in a
  // workgroup barrier:
  //   M(j): S^T of tile j+1 and P.V of tile j-1 (sixteen MFMAs);
  //   V(j): softmax of tile j, store of tile j+3 (loaded during V(j-1)),
  //         loads of tile j+4.
  // Wavefronts 4..7 run one phase behind wavefronts 0..3 (one extra barrier
  // at the start of a window for them, at its end for the others), and each
  // SIMD holds one wavefront of each group, so while one of its wavefronts
  // issues MFMAs the other computes exponentials.  K of tile t is read in
  // M(t-1) of both groups, V of tile t in M(t+1): four K buffers and five V
  // buffers keep every store clear of reads still pending in the lagging
  // group.
  // wavefront-uniform, and visibly so to the compiler (readfirstlane), so
  // the extra barriers below sit behind scalar branches: a wavefront that
  // does not take them never executes them
  const bool lag = __builtin_amdgcn_readfirstlane(wave) >= W / 2;
  for (int wbeg = 0; wbeg < nkv; wbeg += kWinTiles) {
    const int nw = min(kWinTiles, nkv - wbeg);
    win0 = j0 + wbeg;
    {
      const int b0 = win0 * (kKvTile / kPage);
      const int nb = nw * (kKvTile / kPage);
      for (int i = tid; i < nb; i += T) {
        const int j = b0 + i;
        pg_lds[i] = (j < nblk) ? (uint64_t)(uint32_t)bt[j >> ps] * page_bytes +
                                     (uint64_t)((j & pmask) * block_bytes)
                               : 0ull;
      }
      __syncthreads();
    }
    // the first three tiles' loads are all issued before any is stored, so
    // the window start waits on memory once rather than three times
    uint4 rg[NR], r1[NR], r2[NR];
    load_tile(0, rg);
    load_tile(min(1, nw - 1), r1);
    load_tile(min(2, nw - 1), r2);
    store_tile(0, 0, 0, rg);
    if (1 < nw) store_tile(1, 1, 1, r1);
    if (2 < nw) store_tile(2, 2, 2, r2);
    load_tile(min(3, nw - 1), rg);
    __syncthreads();
    qk(0, st_cur);
    if (lag) __syncthreads();
    for (int j = 0; j < nw; ++j) {
      // M(j)
      if (j + 1 < nw) qk((j + 1) % kKBufs, st_next);
      if (j >= 1) pv((j - 1) % kVBufs);
      __syncthreads();
      // V(j)
      softmax(win0 + j);
      if (j + 3 < nw) store_tile(j + 3, (j + 3) % kKBufs, (j + 3) % kVBufs, rg);
      load_tile(min(j + 4, nw - 1), rg);
      st_cur = st_next;
      __syncthreads();
    }
    pv((nw - 1) % kVBufs);  // M(nw): P.V of the last tile
    __syncthreads();
    if (!lag) __syncthreads();
  }

  const f32x2 lh = halves(lsum);
  const float l = lh[0] + lh[1];
  if (!row_valid) return;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  const float row_lse = (l > 0.f) ? (m + fast_log2(l)) * kLn2 : kNegInf;
  if (nsplit > 1) {  // partial of this run: normalised O and its lse
    float* dst = p.tpart_o + (orow * nsplit + split) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int d = 32 * mt + 8 * rb + 4 * half;
        *reinterpret_cast<float4*>(dst + d) =
            make_float4(o[mt][4 * rb] * inv, o[mt][4 * rb + 1] * inv, o[mt][4 * rb + 2] * inv,
                        o[mt][4 * rb + 3] * inv);
      }
    if (half == 0) p.tpart_lse[orow * nsplit + split] = row_lse;
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int d = 32 * mt + 8 * rb + 4 * half;
      const float a0 = o[mt][4 * rb] * inv, a1 = o[mt][4 * rb + 1] * inv;
      const float a2 = o[mt][4 * rb + 2] * inv, a3 = o[mt][4 * rb + 3] * inv;
      if (p.out_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + orow * D + d) =
            make_float4(a0, a1, a2, a3);
      } else {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + orow * D + d) =
            make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
      }
    }
  if (p.lse && half == 0) p.lse[orow] = row_lse;
}

}  // namespace prefill_detail
}  // namespace pa
