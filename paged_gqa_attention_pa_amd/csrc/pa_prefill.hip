// Paged GQA prefill / chunked prefill / mixed batch for gfx950 (bf16 MFMA).
//
// One workgroup = (query tile of one sequence, kv head).  Its Q-block is
// 128 rows: QT = 128 / G query tokens x the G query heads that share the KV
// head (the Q-Block step of the IBM Triton summary's five-step list), row
// r -> token r / G, head r % G; wavefront w owns rows 32w..32w+31 and each
// lane owns one row (lane % 32).  The workgroup walks the sequence's keys in
// tiles of 32 (two pages), up to the causal limit of its last token, staging
// each K and V tile in LDS once for all four wavefronts (FlashAttention-style
// tiling, guide sections "Flash Attention革命" and "Triton实现Flash
// Attention"):
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, K rows from LDS (16-byte reads),
//                 Q^T held in registers; lane l receives 16 keys of row l%32.
//   online softmax in the log2 domain with a lazily raised running max;
//   masked keys (past the context, or after the row's causal position) are
//   removed by select.
//   O^T += V^T P^T  v_mfma_f32_32x32x16_bf16; P (rounded to bf16) is already
//                 in the B-operand layout the S^T result left it in; V^T is
//                 gathered from LDS.  The precise variant splits P into a bf16
//                 high part and a bf16 remainder (two MFMAs), leaving a
//                 relative weight error of about 2^-18 instead of 2^-9.
// Each sequence's query tokens are the last q_len positions of its context:
// query token i sees keys j <= L - q_len + i (bottom-right causal alignment,
// so a chunk attends to its cached prefix in full).  The grid is static:
// x runs over a host bound on query tiles; each workgroup finds its
// sequence by a scan of query_start_loc and surplus workgroups exit.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;   // Q-block rows per workgroup
constexpr int kKvTile = 32;          // keys per inner step
constexpr int kLdsStride = kHeadDim + 8;  // bf16 elements per LDS row (272 B)
constexpr float kLazyThreshold = 8.0f;

// Find (sequence, query tile) of workgroup x: tiles are numbered sequence by
// sequence, ceil(q_len / qt) per sequence.  Returns false for a surplus x.
__device__ bool find_tile(const int32_t* qsl, int num_seqs, int qt, int x, int* seq, int* tile) {
  __shared__ int s_found[2];
  __shared__ int s_wsum[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_found[0] = -1;
  int base = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += 64 * kWaves) {
    const int s = c0 + tid;
    int cnt = 0;
    if (s < num_seqs) cnt = (qsl[s + 1] - qsl[s] + qt - 1) / qt;
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
    for (int w = 0; w < kWaves; ++w) {
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

template <int G, bool PRECISE>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
  constexpr int D = kHeadDim;
  constexpr int QT = kRows / G;
  const int g = blockIdx.y;
  int s, qtile;
  if (!find_tile(p.query_start_loc, p.num_seqs, QT, blockIdx.x, &s, &qtile)) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, half = lane >> 5;
  const int q0 = p.query_start_loc[s];
  const int qlen = p.query_start_loc[s + 1] - q0;
  const int L = p.context_lens[s];
  const int tok0 = qtile * QT;
  const int ntok = min(QT, qlen - tok0);

  // This lane's row.
  const int r = 32 * wave + n;
  const int tl = r / G, h = r % G;
  const bool row_valid = tl < ntok;
  const int qi = tok0 + tl;  // index of the token inside the chunk
  const int key_limit = p.causal ? min(L, L - qlen + qi + 1) : L;  // keys < limit
  const int kv_end = p.causal ? min(L, L - qlen + tok0 + ntok) : L;
  const int nkv = kv_end > 0 ? (kv_end + kKvTile - 1) / kKvTile : 0;

  // Q^T operand: lane holds Q[row][16ks + 8*half .. +8] for ks = 0..7.
  bf16x8 qb[8];
  {
    const uint16_t* qrow = p.q + ((int64_t)(q0 + qi) * p.num_q_heads + g * G + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qb[ks] = row_valid ? as_bf16x8(ld16(qrow + 16 * ks)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kKvTile * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kKvTile * kLdsStride];

  // Tile loader: 32 keys x 16 chunks of 16 bytes, two chunks per thread.
  const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks;
  const uint16_t* kb = p.k_pool + (int64_t)g * p.stride_head;
  const uint16_t* vb = p.v_pool + (int64_t)g * p.stride_head;
  uint4 kreg[2], vreg[2];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int id = tid + 256 * u;
      const int key = j * kKvTile + (id >> 4);
      const int col = (id & 15) * 8;
      if (key < L) {
        const int64_t page = bt[key / kPage];
        const int64_t off = page * p.stride_page + (int64_t)(key % kPage) * p.stride_token + col;
        kreg[u] = ld16(kb + off);
        vreg[u] = ld16(vb + off);
      } else {
        kreg[u] = make_uint4(0, 0, 0, 0);
        vreg[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int id = tid + 256 * u;
      const int idx = (id >> 4) * kLdsStride + (id & 15) * 8;
      *reinterpret_cast<uint4*>(&k_lds[idx]) = kreg[u];
      *reinterpret_cast<uint4*>(&v_lds[idx]) = vreg[u];
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[mt][e] = 0.f;
  float m = kNegInf, lsum = 0.f;

  if (nkv > 0) load_tile(0);
  for (int j = 0; j < nkv; ++j) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (j + 1 < nkv) load_tile(j + 1);

    // S^T = K Q^T over D = 128 (8 steps of 16).
    f32x16 st;
#pragma unroll
    for (int e = 0; e < 16; ++e) st[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 a = *reinterpret_cast<const uint4*>(&k_lds[n * kLdsStride + 16 * ks + 8 * half]);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qb[ks], st, 0, 0, 0);
    }

    // Register e holds key 8*(e/4) + 4*half + e%4 of this tile, row n.
    const int kbase = j * kKvTile + 4 * half;
    float x[16];
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kbase + 8 * (e >> 2) + (e & 3);
      x[e] = (key < key_limit) ? st[e] * p.scale_log2 : kNegInf;
      tmax = fmaxf(tmax, x[e]);
    }
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const bool need = tmax > m + kLazyThreshold;
    if (wave_any(need)) {
      const float m_new = need ? tmax : m;
      const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[mt][e] *= alpha;
    }
    const float m_use = (m == kNegInf) ? 0.f : m;
    uint32_t pk[8], pl[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = fast_exp2(x[e] - m_use);
      const float p1 = fast_exp2(x[e + 1] - m_use);
      psum += p0 + p1;
      pk[e >> 1] = pack_bf16x2(p0, p1);
      if constexpr (PRECISE) {
        pl[e >> 1] = pack_bf16x2(p0 - bf16lo(pk[e >> 1]), p1 - bf16hi(pk[e >> 1]));
      }
    }
    lsum += psum;

    // O^T += V^T P^T: two k-steps of 16 keys, four 32-dim M tiles.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pk[4 * kk], pk[4 * kk + 1],
                                                              pk[4 * kk + 2], pk[4 * kk + 3]));
      bf16x8 pbl;
      if constexpr (PRECISE)
        pbl = __builtin_bit_cast(bf16x8, make_uint4(pl[4 * kk], pl[4 * kk + 1], pl[4 * kk + 2],
                                                    pl[4 * kk + 3]));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int d = 32 * mt + n;
        uint16_t vv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = 16 * kk + 8 * (i >> 2) + 4 * half + (i & 3);
          vv[i] = v_lds[key * kLdsStride + d];
        }
        const uint4 va = make_uint4((uint32_t)vv[0] | ((uint32_t)vv[1] << 16),
                                    (uint32_t)vv[2] | ((uint32_t)vv[3] << 16),
                                    (uint32_t)vv[4] | ((uint32_t)vv[5] << 16),
                                    (uint32_t)vv[6] | ((uint32_t)vv[7] << 16));
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), pb, o[mt], 0, 0, 0);
        if constexpr (PRECISE)
          o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), pbl, o[mt], 0, 0, 0);
      }
    }
  }

  const float l = lsum + shfl_xor(lsum, 32);
  if (!row_valid) return;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  const int64_t orow = (int64_t)(q0 + qi) * p.num_q_heads + g * G + h;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
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
  if (p.lse && half == 0) p.lse[orow] = (l > 0.f) ? (m + fast_log2(l)) * kLn2 : kNegInf;
}

}  // namespace

template <bool PRECISE>
hipError_t launch_prefill_t(const PrefillParams& p, int group, dim3 grid, hipStream_t stream) {
  dim3 block(256);
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<1, PRECISE>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<2, PRECISE>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<4, PRECISE>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<8, PRECISE>), grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL((prefill_kernel<16, PRECISE>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int group, int grid_x, bool precise_p,
                          hipStream_t stream) {
  if (grid_x <= 0) return hipSuccess;
  dim3 grid(grid_x, p.num_kv_heads, 1);
  return precise_p ? launch_prefill_t<true>(p, group, grid, stream)
                   : launch_prefill_t<false>(p, group, grid, stream);
}

}  // namespace pa
