// Paged GQA decode with split-KV, for gfx950.
//
// One workgroup = (split, kv head, sequence); four wavefronts stream the
// split's 16-key tiles (tile t = page t, page size 16) round-robin, each with
// its own online-softmax state, and merge at the end through LDS.
//
// Per tile and wavefront:
//   * K is read straight from HBM into the A operand of one
//     v_mfma_f32_16x16x32_bf16 per 32 dims (16-byte loads: lane l reads 16
//     bytes of the K row of key sigma(l % 16)), and the query heads of this
//     KV head form the B operand, repeated across the 16 columns when G < 16
//     (the Q-Block grouping of the IBM Triton summary's five-step list: K
//     and V are read once for all G heads).  The result S^T lands so that
//     lane (c, n) holds head n % G for keys c, c+4, c+8, c+12 of the tile.
//   * Online softmax in the log2 domain (scale*log2(e) folded into one
//     multiply); the running maximum is raised lazily, only when a tile's
//     maximum exceeds it by more than 8, so exponentials stay below 2^8 and
//     the accumulator is rescaled rarely.  The recurrence is the m / l update
//     of the guide's "Flash Attention革命" section.
//   * P.V in fp32 on the VALU: lane (c, n) owns dims 8n..8n+7 of keys
//     c + 4i; V rows are 16-byte coalesced loads (four full 256-byte rows per
//     instruction).  P stays fp32, so no rounding is added to the weights.
// Masked keys (past the context, or stale NaN slots of the last page) are
// removed by select, never by arithmetic.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
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

template <int G>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  constexpr int D = kHeadDim;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int c = lane >> 4;  // key group: keys c + 4i of a tile
  const int n = lane & 15;  // MFMA column; head n % G; dims 8n..8n+7 in P.V
  const int hl = n % G;

  const int L = p.context_lens[b];
  const int ntiles = (L + kDecodeTile - 1) / kDecodeTile;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(t_begin + p.tiles_per_split, ntiles);

  // B operand: this KV head's query heads (column n -> head n % G).
  const uint16_t* qrow = p.q + ((int64_t)b * p.num_q_heads + g * G + hl) * D;
  bf16x8 qb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qb[j] = as_bf16x8(ld16(qrow + 32 * j + 8 * c));

  const int ktok = (n >> 2) + 4 * (n & 3);  // sigma: MFMA row -> key in tile
  const uint16_t* kbase = p.k_pool + (int64_t)g * p.stride_head + (int64_t)ktok * p.stride_token + 8 * c;
  const uint16_t* vbase = p.v_pool + (int64_t)g * p.stride_head + (int64_t)c * p.stride_token + 8 * n;
  const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks;

  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m = kNegInf;  // running log2-domain max for head hl
  float lsum = 0.f;   // partial softmax denominator (this lane's keys)

  for (int t = t_begin + wave; t < t_end; t += kWaves) {
    const int64_t page = bt[t];
    const uint16_t* kp = kbase + page * p.stride_page;
    const uint16_t* vp = vbase + page * p.stride_page;
    uint4 kr[4], vr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kr[j] = ld16(kp + 32 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = ld16(vp + (int64_t)(4 * i) * p.stride_token);

    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[j]), qb[j], s, 0, 0, 0);

    const int key0 = t * kDecodeTile + c;
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (key0 + 4 * i < L) ? s[i] * p.scale_log2 : kNegInf;
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
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(x[i] - m);
    lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    if (t * kDecodeTile + kDecodeTile > L) {  // last tile: drop stale V rows
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + 4 * i >= L) vr[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[8];
      v[0] = bf16lo(vr[i].x); v[1] = bf16hi(vr[i].x);
      v[2] = bf16lo(vr[i].y); v[3] = bf16hi(vr[i].y);
      v[4] = bf16lo(vr[i].z); v[5] = bf16hi(vr[i].z);
      v[6] = bf16lo(vr[i].w); v[7] = bf16hi(vr[i].w);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = head_bcast<G>(pr[i], h, lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, v[e], acc[h][e]);
      }
    }
  }

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

  // Merge the four wavefronts through LDS.
  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  if (c == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(&sm_acc[wave][h][8 * n]);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
    if (n < G) {
      sm_m[wave][n] = m;
      sm_l[wave][n] = lsum;
    }
  }
  __syncthreads();

  const int S = p.num_splits;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float o = 0.f, l = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm_m[w][h];
        if (mw != kNegInf) {
          const float e = fast_exp2(mw - M);
          o = fmaf(e, sm_acc[w][h][d], o);
          l = fmaf(e, sm_l[w][h], l);
        }
      }
      o = o / l;
    }
    const float lse_nat = (M == kNegInf) ? kNegInf : (M + fast_log2(l)) * kLn2;
    const int64_t row = (int64_t)b * p.num_q_heads + g * G + h;
    if (S == 1) {
      if (p.out_f32)
        reinterpret_cast<float*>(p.out)[row * D + d] = o;
      else
        reinterpret_cast<uint16_t*>(p.out)[row * D + d] = f2bf(o);
      if (p.lse && d == 0) p.lse[row] = lse_nat;
    } else {
      p.part_o[(row * S + split) * D + d] = o;
      if (d == 0) p.part_lse[row * S + split] = lse_nat;
    }
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int group, hipStream_t stream) {
  dim3 grid(p.num_splits, p.num_kv_heads, p.num_seqs);
  dim3 block(64 * kWaves);
  switch (group) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL(decode_split_kernel<8>, grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL(decode_split_kernel<16>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
