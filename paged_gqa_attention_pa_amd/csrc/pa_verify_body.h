// Short query runs over the paged cache (speculative-decode verification:
// a few causal query tokens per sequence, the speculative-decoding feature of
// the IBM Triton summary's model-feature list), for gfx950.
//
// A (sequence, kv head) unit is q_s tokens x G query heads = R <= 16*RB rows,
// and the whole of it is one Q-block (the Q-Block step of the same summary's
// five-step list, stretched over tokens as well as heads): K and V are read
// once for all R rows.  The work split is the decode one: W wavefronts take
// a piece's 16-key tiles (16 slots of a page each) round-robin, each with its own
// online-softmax state, and merge through LDS at the end.
//
// Per tile and wavefront:
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16, one per 32 dims and 16-row
//     block: K comes straight from HBM into the A operand (lane (c, n) reads
//     dims 8c..8c+7 of every 32 of key n's row), the Q-block is the B operand
//     (column 16*rb + n is row r = i*G + h: token i, head h).  Lane (c, n)
//     ends with keys 4c..4c+3 of column n.
//   * Online softmax per column in the log2 domain, lazily raised maximum
//     (as the decode body); a column past its causal limit is masked by
//     select.  P is rounded to bf16 (fp32 outputs: bf16 high part plus a bf16
//     remainder, two MFMAs).
//   * O^T += V^T P^T with v_mfma_f32_16x16x16_bf16 per 16-dim block: the S^T
//     accumulator layout (keys 4c..4c+3, column n) is already the B operand,
//     and V^T comes from the wavefront's V tile in LDS through
//     ds_read_b64_tr_b16 (V rows arrive from HBM as 16-byte row pieces and
//     are written row-major; V rows past the context are zeroed first).
//   * A ring of DEPTH tiles of K and V loads keeps two tiles in flight.
#pragma once

#include "pa_decode_body.h"

namespace pa {
namespace verify_detail {

using decode_detail::EvenPiece;
using decode_detail::kLazyThreshold;
using decode_detail::readlane;

// bf16 per V row in LDS: D of data + 16 of pad (the transposing reads of
// 16 rows then fall on two bank rounds)
template <int D>
constexpr int v_row() {
  return D + 16;
}

// LDS floats verify_body needs from its caller: one V tile per wavefront
// during the loop, then one 16-column block of O per wavefront for the merge.
template <int W, int D>
constexpr int verify_smem_floats() {
  constexpr int vtiles = W * 16 * v_row<D>() / 2;
  constexpr int merge = W * 16 * D;
  return vtiles > merge ? vtiles : merge;
}

// Rows (token, head) of a unit whose query run is R <= 16*RB long.
__device__ __forceinline__ int64_t unit_row(const DecodeParams& p, int q0, int g, int G,
                                            int r) {
  return (int64_t)(q0 + r / G) * p.num_q_heads + g * G + r % G;
}

// One workgroup of W wavefronts: the piece ev of unit (sequence b, kv head g),
// head dimension D (64, 128 or 256).
// sm_buf: verify_smem_floats<W, D>() floats of LDS, 16-byte aligned.
template <int G, int RB, int W, bool PRECISE, int D = kHeadDim>
__device__ __forceinline__ void verify_body(const DecodeParams& p, int g, int b, float* sm_buf,
                                            EvenPiece ev) {
  static_assert(D == 64 || D == 128 || D == 256, "head dims built");
  constexpr int KS = D / 32;   // k-steps of the S^T MFMA (32 dims each)
  constexpr int DB = D / 16;   // 16-dim blocks of the P.V MFMA
  constexpr int NV = D / 32;   // 16-byte V loads per lane and tile
  constexpr int CH = D / 8;    // 16-byte chunks per V row
  constexpr int kVRow = v_row<D>();
  // Four or eight row blocks: RB / 2 wavefronts share one stream of tiles
  // (the later reads of a tile are L2 hits) and each keeps two of the row
  // blocks, so its registers are those of two row blocks.
  constexpr int WPS = RB >= 4 ? RB / 2 : 1;  // wavefronts per tile stream
  static_assert(W % WPS == 0, "row blocks per workgroup");
  constexpr bool kPairs = WPS > 1;
  constexpr int RBW = RB / WPS;  // row blocks of one wavefront
  constexpr int WS = W / WPS;    // tile streams of the workgroup
  // tiles per wavefront ring (registers bound it)
  constexpr int DEPTH = (RBW >= 2 || D >= 256) ? 2 : 3;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int strm = wave / WPS;           // this wavefront's tile stream
  const int rb0 = (wave % WPS) * RBW;    // its first row block
  const int lane = tid & 63;
  const int c = lane >> 4;
  const int n = lane & 15;
  // query_start_loc null: sequence b owns token b (decode layout)
  const int q0 = p.query_start_loc ? p.query_start_loc[b] : b;
  const int qn = p.query_start_loc ? p.query_start_loc[b + 1] - q0 : 1;
  const int R = qn * G;
  if (qn <= 0 || R > 16 * RB) return;  // no rows, or above the host bound

  // Q-block (B operands) and this wave's first 64 page ids, before the
  // context length arrives.
  bf16x8 qb[RBW][KS];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = 16 * (rb0 + rb) + n;
    if (r < R) {
      const uint16_t* qrow = p.q + unit_row(p, q0, g, G, r) * D + 8 * c;
#pragma unroll
      for (int j = 0; j < KS; ++j) qb[rb][j] = as_bf16x8(ld16(qrow + 32 * j));
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) qb[rb][j] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  const int t_begin = ev.t_begin;
  // 16-key tile t lies in block-table entry t >> page_shift, 16 * (t & pmask)
  // slots into that page
  const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks;
  const int ps = p.page_shift, pmask = (1 << p.page_shift) - 1;
  const int tok16 = 16 * (int)p.stride_token;  // < 2^31: a page spans < 2^31 elements
  const int t_first = t_begin + strm + WS * lane;
  int pages = ((t_first >> ps) < p.max_blocks) ? bt[t_first >> ps] : 0;

  const int L = p.context_lens[b];
  const int t_end = ev.t_end;
  const int nt =
      (t_end - t_begin - strm + WS - 1) / WS > 0 ? (t_end - t_begin - strm + WS - 1) / WS : 0;

  // keys < lim[rb] are allowed in column 16*rb + n; every column is limited
  // from key lim_lo on
  int lim[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = 16 * (rb0 + rb) + n;
    lim[rb] = (p.causal && r < R) ? L - qn + r / G + 1 : L;
  }
  const int lim_lo = p.causal ? L - qn + 1 : L;

  const uint16_t* kbase = p.k_pool + (int64_t)g * p.stride_head + (int64_t)n * p.stride_token + 8 * c;
  // V load u of this lane: chunk (64u + lane) of the tile's 16 x CH row chunks
  const uint16_t* vbase = p.v_pool + (int64_t)g * p.stride_head +
                          (int64_t)(lane / CH) * p.stride_token + 8 * (lane % CH);
  uint16_t* vt = reinterpret_cast<uint16_t*>(sm_buf) + wave * 16 * kVRow;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  // transposing read of lane (c, n): row 4c + n/4, dims 4(n%4) (+16 per block)
  const int tr_off = (4 * c + (n >> 2)) * kVRow + 4 * (n & 3);

  auto fetch_pages = [&](int chunk) {
    const int i = lane + 64 * chunk;
    pages = (i < nt) ? bt[(t_begin + strm + WS * i) >> ps] : 0;
  };
  int chunk_base = 0;  // first tile index (of this stream's list) of the current chunk
  auto issue = [&](int i, uint4 (&kr)[KS], uint4 (&vr)[NV]) {
    const int64_t page = readlane(pages, i & 63);
    const int t = t_begin + strm + WS * (chunk_base + i);
    const int64_t off = page * p.stride_page + (int64_t)((t & pmask) * tok16);
    const uint16_t* kp = kbase + off;
    const uint16_t* vp = vbase + off;
#pragma unroll
    for (int j = 0; j < KS; ++j) kr[j] = ld16(kp + 32 * j);
#pragma unroll
    for (int u = 0; u < NV; ++u) vr[u] = ld16(vp + (int64_t)(64 / CH * u) * p.stride_token);
  };

  f32x4 acc[DB][RBW];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) acc[db][rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m[RBW], lsum[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    m[rb] = kNegInf;
    lsum[rb] = 0.f;
  }

  uint4 kr[DEPTH][KS], vr[DEPTH][NV];

  auto process = [&](uint4 (&kc)[KS], uint4 (&vc)[NV], int i) {
    const int t = t_begin + strm + WS * i;
    f32x4 s[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      s[rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j)
        s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[j]), qb[rb][j], s[rb], 0, 0, 0);
    }
    const int key0 = t * kDecodeTile + 4 * c;
    const bool edge = t * kDecodeTile + kDecodeTile > lim_lo;
    float x[RBW][4];
    bool need_any = false;
    float tmax[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[rb][e] = s[rb][e] * p.scale_log2;
        if (edge && key0 + e >= lim[rb]) x[rb][e] = kNegInf;
      }
      float mx = fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3]));
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      tmax[rb] = mx;
      need_any |= mx > m[rb] + kLazyThreshold;
    }
    if (wave_any(need_any)) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        const bool need = tmax[rb] > m[rb] + kLazyThreshold;
        const float alpha = need ? fast_exp2(m[rb] - tmax[rb]) : 1.f;  // 0 on a first raise
        m[rb] = need ? tmax[rb] : m[rb];
        lsum[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][rb] *= alpha;
      }
    }

    // P (B operands of the P.V MFMA); a column with no allowed key yet keeps
    // m = -inf and gets P = 0
    i16x4 ph[RBW], pl[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      const float mm = m[rb] == kNegInf ? 0.f : m[rb];
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pr[e] = fast_exp2(x[rb][e] - mm);
      const uint32_t w0 = pack_bf16x2(pr[0], pr[1]);
      const uint32_t w1 = pack_bf16x2(pr[2], pr[3]);
      ph[rb] = __builtin_bit_cast(i16x4, make_uint2(w0, w1));
      if constexpr (PRECISE) {
        const uint32_t l0 = pack_bf16x2(pr[0] - bf16lo(w0), pr[1] - bf16hi(w0));
        const uint32_t l1 = pack_bf16x2(pr[2] - bf16lo(w1), pr[3] - bf16hi(w1));
        pl[rb] = __builtin_bit_cast(i16x4, make_uint2(l0, l1));
        lsum[rb] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      } else {
        lsum[rb] = add_bf16x2(w1, add_bf16x2(w0, lsum[rb]));
      }
    }

    if (t * kDecodeTile + kDecodeTile > L) {  // last tile: drop stale V rows
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (t * kDecodeTile + (64 * u + lane) / CH >= L) vc[u] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < NV; ++u)
      *reinterpret_cast<uint4*>(vt + ((64 * u + lane) / CH) * kVRow + 8 * (lane % CH)) = vc[u];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + tr_off + 16 * db));
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        acc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph[rb], acc[db][rb], 0, 0, 0);
        if constexpr (PRECISE)
          acc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl[rb], acc[db][rb], 0, 0, 0);
      }
    }
  };

  // The decode body's software pipeline: chunks of 64 tiles, tile i of a
  // chunk in ring slot i % DEPTH, no load under a branch.
  for (int cb = 0; cb < nt; cb += 64) {
    const int nc = min(64, nt - cb);
    chunk_base = cb;
    if (cb > 0) fetch_pages(cb >> 6);
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) issue(min(d, nc - 1), kr[d], vr[d]);
    int i0 = 0;
    for (; i0 + DEPTH <= nc; i0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        constexpr int kAhead = DEPTH - 1;
        issue(min(i0 + d + kAhead, nc - 1), kr[(d + kAhead) % DEPTH], vr[(d + kAhead) % DEPTH]);
        process(kr[d], vr[d], cb + i0 + d);
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
      if (i0 + d < nc) process(kr[d], vr[d], cb + i0 + d);
  }

#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    lsum[rb] += shfl_xor(lsum[rb], 16);
    lsum[rb] += shfl_xor(lsum[rb], 32);
  }

  // Merge the W wavefronts, one 16-column block at a time (a wavefront that
  // does not hold a block reports m = -inf for it and is skipped).
  __shared__ float sm_m[W][16 * RB];
  __shared__ float sm_l[W][16 * RB];
  if (c == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool mine = rb >= rb0 && rb < rb0 + RBW;
      sm_m[wave][16 * rb + n] = mine ? m[rb % RBW] : kNegInf;
      sm_l[wave][16 * rb + n] = mine ? lsum[rb % RBW] : 0.f;
    }
  }
  const int S = ev.slots;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (16 * rb >= R) break;
    __syncthreads();  // the V tiles, or the previous block, are no longer read
    float* so = sm_buf + wave * 16 * D;
    if (rb >= rb0 && rb < rb0 + RBW) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(so + n * D + 16 * db + 4 * c) = acc[db][rb % RBW];
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * (D / 4); idx += 64 * W) {
      const int col = idx / (D / 4);
      const int d0 = 4 * (idx % (D / 4));
      const int r = 16 * rb + col;
      if (r >= R) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][r]);
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      float l = 0.f;
      if (M != kNegInf) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float mw = sm_m[w][r];
          if (mw != kNegInf) {
            const float e = fast_exp2(mw - M);
            o += e * *reinterpret_cast<const f32x4*>(sm_buf + (w * 16 + col) * D + d0);
            l = fmaf(e, sm_l[w][r], l);
          }
        }
        o /= l;
      }
      const float lse_nat = (M == kNegInf) ? kNegInf : (M + fast_log2(l)) * kLn2;
      const int64_t row = unit_row(p, q0, g, G, r);
      if (ev.direct) {
        if (p.out_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + row * D + d0) = o;
        } else {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * D + d0) =
              make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
        if (p.lse && d0 == 0) p.lse[row] = lse_nat;
      } else {
        *reinterpret_cast<f32x4*>(p.part_o + (row * S + ev.slot) * D + d0) = o;
        if (d0 == 0) p.part_lse[row * S + ev.slot] = lse_nat;
      }
    }
  }
}

}  // namespace verify_detail
}  // namespace pa
