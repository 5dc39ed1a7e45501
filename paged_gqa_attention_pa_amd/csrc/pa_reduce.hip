// Log-sum-exp merge of split-KV partials (the exact merge behind the
// parallel tiled softmax of the IBM Triton summary's five-step list; the
// algebra is that of the online-softmax statistics m and l, guide section
// "Flash Attention革命"):
//   M = max_k lse_k, w_k = exp(lse_k - M),
//   O = sum_k w_k O_k / sum_k w_k,  LSE = M + ln sum_k w_k,
// and O = 0, LSE = -inf when every split is empty.  Empty splits (lse = -inf)
// get weight 0 without evaluating -inf - (-inf).
//
// One 256-thread workgroup per row: the weights go to LDS once, then thread
// (group, item) accumulates dims 4*item..4*item+3 over the splits k = group,
// group + groups, ... with batches of eight independent 16-byte loads, and
// the groups are summed through LDS.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_prefill_body.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kPre = 4;  // partial-O loads per thread issued up front
constexpr int kMaxUnitRows = 64;  // rows of one short-run unit (q_s * G)
// Short-run merges: one workgroup per unit when the batch has at least this
// many rows, else one per (unit, row).  Measured on gfx950: 512 units of 16
// rows (2-3 pieces each) merge in 5.5 us per unit against 23.8 us per row;
// one unit of 32 rows in 65 pieces in 24.7 us per row against 47.9 us (whole
// decode step) per unit.
constexpr int kUnitMergeMinRows = 1024;

__device__ float block_reduce(float v, bool is_max, float* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, scratch[w]) : r + scratch[w];
  return r;
}

__global__ __launch_bounds__(kThreads) void splitkv_reduce_kernel(ReduceParams p) {
  __shared__ float w_lds[kReduceMaxSplits];
  __shared__ __attribute__((aligned(16))) float red[kThreads * 4];
  __shared__ float scratch[kThreads / 64];
  int row = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t orow = row;
  int b = row / p.num_q_heads;  // sequence of the row
  if (p.unit_rows) {
    // short-run partials: workgroup (unit, r) merges row r of the (sequence,
    // kv head) unit, token r / G, head g*G + r % G
    const int G = p.group;
    const int Hkv = p.num_q_heads / G;
    const int u = blockIdx.x;
    b = u / Hkv;
    const int g = u % Hkv;
    const int q0 = p.query_start_loc ? p.query_start_loc[b] : b;
    const int qn = p.query_start_loc ? p.query_start_loc[b + 1] - q0 : 1;
    const int r = blockIdx.y;
    if (r >= qn * G) return;
    row = (q0 + r / G) * p.num_q_heads + g * G + r % G;
    orow = row;
  } else if (p.query_start_loc) {  // mixed batch: merge the single-token sequences only
    const int s = row / p.num_q_heads;
    const int q0 = p.query_start_loc[s];
    if (p.query_start_loc[s + 1] - q0 != 1) return;
    orow = (int64_t)q0 * p.num_q_heads + row % p.num_q_heads;
  }
  const int stride = p.num_splits;  // partial slots per row
  int S = stride;                   // slots in use
  const int D = p.head_dim;
  if (p.piece_counts) {
    // even-work decode grid: an empty context has no pieces (O = 0,
    // lse = -inf); a unit of one piece was written directly
    const int u = b * (p.num_q_heads / p.group) + (row % p.num_q_heads) / p.group;
    if (p.context_lens[b] <= 0) {
      for (int d = tid; d < D; d += kThreads) {
        if (p.out_f32)
          reinterpret_cast<float*>(p.out)[orow * D + d] = 0.f;
        else
          reinterpret_cast<uint16_t*>(p.out)[orow * D + d] = 0;
      }
      if (p.lse && tid == 0) p.lse[orow] = kNegInf;
      return;
    }
    S = min(p.piece_counts[u], stride);
    if (S <= 1) return;
  }
  const float* lse_row = p.part_lse + (int64_t)row * stride;

  // Up to kPre * (threads / (D/4)) splits: each thread's partial-O loads are
  // issued here, before the weights are known, so the workgroup waits on
  // memory once rather than twice.
  const int items = D / 4;
  const bool pre = items <= kThreads && S <= (kThreads / items) * kPre;
  float4 pv[kPre];
  if (pre) {
    const int groups = kThreads / items, item = tid % items, grp = tid / items;
    const float* src = p.part_o + (int64_t)row * stride * D + 4 * item;
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int k = grp + u * groups;
      pv[u] = (grp < groups && k < S) ? *reinterpret_cast<const float4*>(src + (int64_t)k * D)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }

  float M = kNegInf;
  for (int k = tid; k < S; k += kThreads) {
    const float l = lse_row[k];
    w_lds[k] = l;
    M = fmaxf(M, l);
  }
  M = block_reduce(M, true, scratch);
  float wsum = 0.f;
  if (M != kNegInf) {
    for (int k = tid; k < S; k += kThreads) {
      const float l = w_lds[k];
      const float w = (l == kNegInf) ? 0.f : fast_exp2((l - M) * kLog2e);
      w_lds[k] = w;
      wsum += w;
    }
  }
  wsum = block_reduce(wsum, false, scratch);  // also orders the w_lds writes
  const float inv = (M != kNegInf) ? 1.f / wsum : 0.f;

  for (int base = 0; base < items; base += kThreads) {
    const int chunk = min(kThreads, items - base);
    const int groups = kThreads / chunk;
    const int item = base + tid % chunk;
    const int grp = tid / chunk;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (pre && grp < groups && M != kNegInf) {
#pragma unroll
      for (int u = 0; u < kPre; ++u) {
        const int k = grp + u * groups;
        if (k < S) {
          const float w = w_lds[k];
          const bool on = w != 0.f;
          o.x = fmaf(w, on ? pv[u].x : 0.f, o.x);
          o.y = fmaf(w, on ? pv[u].y : 0.f, o.y);
          o.z = fmaf(w, on ? pv[u].z : 0.f, o.z);
          o.w = fmaf(w, on ? pv[u].w : 0.f, o.w);
        }
      }
    } else if (grp < groups && M != kNegInf) {
      const float* src = p.part_o + (int64_t)row * stride * D + 4 * item;
      // Eight independent loads per batch; an empty split (weight 0) may hold
      // stale values, so its contribution is selected away, not multiplied.
      int k = grp;
      for (; k + 7 * groups < S; k += 8 * groups) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = *reinterpret_cast<const float4*>(src + (int64_t)(k + u * groups) * D);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float w = w_lds[k + u * groups];
          const bool on = w != 0.f;
          o.x = fmaf(w, on ? v[u].x : 0.f, o.x);
          o.y = fmaf(w, on ? v[u].y : 0.f, o.y);
          o.z = fmaf(w, on ? v[u].z : 0.f, o.z);
          o.w = fmaf(w, on ? v[u].w : 0.f, o.w);
        }
      }
      for (; k < S; k += groups) {
        const float w = w_lds[k];
        const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)k * D);
        const bool on = w != 0.f;
        o.x = fmaf(w, on ? v.x : 0.f, o.x);
        o.y = fmaf(w, on ? v.y : 0.f, o.y);
        o.z = fmaf(w, on ? v.z : 0.f, o.z);
        o.w = fmaf(w, on ? v.w : 0.f, o.w);
      }
    }
    __syncthreads();
    if (grp < groups) *reinterpret_cast<float4*>(&red[4 * (grp * chunk + tid % chunk)]) = o;
    __syncthreads();
    if (tid < chunk) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int q = 0; q < groups; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&red[4 * (q * chunk + tid)]);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      acc.x *= inv; acc.y *= inv; acc.z *= inv; acc.w *= inv;
      const int64_t off = orow * D + 4 * (base + tid);
      if (p.out_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + off) = acc;
      } else {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + off) =
            make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
      }
    }
  }
  if (p.lse && tid == 0) p.lse[orow] = (M == kNegInf) ? kNegInf : M + fast_log2(wsum) * kLn2;
}

// Merge of the short-run path's pieces: one workgroup per (sequence, kv head)
// unit, so a row's sequence is the workgroup's and no search is needed.  The
// unit's rows r = 0 .. q_s*G-1 (token r / G, head g*G + r % G) go eight at a
// time over the workgroup, 32 lanes per row with 4 dims each; every lane
// reads the row's piece lse values itself (one broadcast load each) and its
// own 16 bytes of every piece.  Units written in one piece are skipped; an
// empty context gives O = 0, lse = -inf.
__global__ __launch_bounds__(kThreads) void unit_merge_kernel(ReduceParams p) {
  constexpr int kRowsPerPass = kThreads / 32;
  const int G = p.group;
  const int Hkv = p.num_q_heads / G;
  const int u = blockIdx.x;
  const int b = u / Hkv, g = u % Hkv;
  // query_start_loc null: sequence b owns token b (decode layout)
  const int q0 = p.query_start_loc ? p.query_start_loc[b] : b;
  const int qn = p.query_start_loc ? p.query_start_loc[b + 1] - q0 : 1;
  const int R = qn * G;
  if (qn <= 0 || R > kMaxUnitRows) return;
  const int L = p.context_lens[b];
  const int stride = p.num_splits;
  const int count = p.piece_counts[u];  // stale for an empty context: not used then
  const int pieces = L > 0 ? min(count, stride) : 0;
  if (L > 0 && pieces <= 1) return;
  const int D = p.head_dim;
  const int item = threadIdx.x & 31;
  for (int r = threadIdx.x >> 5; r < R; r += kRowsPerPass) {
    const int64_t row = (int64_t)(q0 + r / G) * p.num_q_heads + g * G + r % G;
    const float* lr = p.part_lse + row * stride;
    const float* po = p.part_o + row * stride * D;
    for (int d0 = 4 * item; d0 < D; d0 += 128) {
      // the first four pieces' lse and partial loads go out together
      float l4[4];
      float4 v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        l4[j] = j < pieces ? lr[j] : kNegInf;
        v4[j] = j < pieces ? *reinterpret_cast<const float4*>(po + (int64_t)j * D + d0)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float M = fmaxf(fmaxf(l4[0], l4[1]), fmaxf(l4[2], l4[3]));
      for (int k = 4; k < pieces; ++k) M = fmaxf(M, lr[k]);
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      float wsum = 0.f;
      if (M != kNegInf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float w = (l4[j] == kNegInf) ? 0.f : fast_exp2((l4[j] - M) * kLog2e);
          const bool on = w != 0.f;
          wsum += w;
          o.x = fmaf(w, on ? v4[j].x : 0.f, o.x);
          o.y = fmaf(w, on ? v4[j].y : 0.f, o.y);
          o.z = fmaf(w, on ? v4[j].z : 0.f, o.z);
          o.w = fmaf(w, on ? v4[j].w : 0.f, o.w);
        }
        int k = 4;
        for (; k + 4 <= pieces; k += 4) {  // four independent loads in flight
          float4 v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            v[j] = *reinterpret_cast<const float4*>(po + (int64_t)(k + j) * D + d0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float l = lr[k + j];
            const float w = (l == kNegInf) ? 0.f : fast_exp2((l - M) * kLog2e);
            const bool on = w != 0.f;
            wsum += w;
            o.x = fmaf(w, on ? v[j].x : 0.f, o.x);
            o.y = fmaf(w, on ? v[j].y : 0.f, o.y);
            o.z = fmaf(w, on ? v[j].z : 0.f, o.z);
            o.w = fmaf(w, on ? v[j].w : 0.f, o.w);
          }
        }
        for (; k < pieces; ++k) {
          const float4 v = *reinterpret_cast<const float4*>(po + (int64_t)k * D + d0);
          const float l = lr[k];
          const float w = (l == kNegInf) ? 0.f : fast_exp2((l - M) * kLog2e);
          const bool on = w != 0.f;
          wsum += w;
          o.x = fmaf(w, on ? v.x : 0.f, o.x);
          o.y = fmaf(w, on ? v.y : 0.f, o.y);
          o.z = fmaf(w, on ? v.z : 0.f, o.z);
          o.w = fmaf(w, on ? v.w : 0.f, o.w);
        }
        const float inv = 1.f / wsum;
        o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
      }
      const int64_t off = row * D + d0;
      if (p.out_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + off) = o;
      } else {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + off) =
            make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
      }
      if (p.lse && d0 == 0)
        p.lse[row] = (M == kNegInf) ? kNegInf : M + fast_log2(wsum) * kLn2;
    }
  }
}

// Merge of split query tiles.  Workgroup (kv head g, tile x) finds its tile
// as the prefill workgroups do, so rows of single-token sequences that ran as
// decode workgroups are never touched.  Its rows r = 0 .. ntok*G-1 (token
// r / G, head g*G + r % G) are spread over the eight wavefronts; 32 lanes
// cover one row's 128 dims with 16-byte loads, so a wavefront merges two
// rows per step and keeps four steps (eight rows) of loads in flight.
constexpr int kMergeRowsPerIter = 8;

template <int S, int D>
__global__ __launch_bounds__(prefill_detail::kThreads) void tile_merge_kernel(TileMergeParams p,
                                                                             int nx) {
  using prefill_detail::find_tile;
  constexpr int DPL = D / 32;  // dims per lane: 32 lanes cover a row
  // rows in flight per wavefront step (two per row pair of half-wavefronts);
  // fewer at head dim 256, whose rows are twice as many registers
  constexpr int RPI = DPL == 8 ? 2 : kMergeRowsPerIter;
  const int g = blockIdx.x % p.num_kv_heads;
  const int x = nx - 1 - blockIdx.x / p.num_kv_heads;
  int s, qtile;
  if (!find_tile(p.query_start_loc, p.num_seqs, p.q_tile, x, p.decode_rows_apart != 0, &s,
                 &qtile))
    return;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int q0 = p.query_start_loc[s];
  const int qlen = p.query_start_loc[s + 1] - q0;
  const int tok0 = qtile * p.q_tile;
  const int nrows = min(p.q_tile, qlen - tok0) * G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane >> 5, dl = lane & 31;
  const int rows_per_wave = (nrows + prefill_detail::kWaves - 1) / prefill_detail::kWaves;
  const int r_begin = wave * rows_per_wave;
  const int r_end = min(nrows, r_begin + rows_per_wave);
  for (int r0 = r_begin; r0 < r_end; r0 += RPI) {
    int64_t orow[RPI / 2];
    bool valid[RPI / 2];
    float M[RPI / 2];
#pragma unroll
    for (int u = 0; u < RPI / 2; ++u) {
      const int r = r0 + 2 * u + sub;
      valid[u] = r < r_end;
      const int rr = valid[u] ? r : r_begin;
      orow[u] = (int64_t)(q0 + tok0 + rr / G) * p.num_q_heads + g * G + rr % G;
      M[u] = kNegInf;
    }
    float lse_v[RPI / 2][S];
    float v[RPI / 2][S][DPL];
#pragma unroll
    for (int u = 0; u < RPI / 2; ++u)
#pragma unroll
      for (int k = 0; k < S; ++k) {
        lse_v[u][k] = p.tpart_lse[orow[u] * S + k];
        const float* src = p.tpart_o + (orow[u] * S + k) * D + DPL * dl;
        if constexpr (DPL == 8) {
          const float4 t0 = *reinterpret_cast<const float4*>(src);
          const float4 t1 = *reinterpret_cast<const float4*>(src + 4);
          v[u][k][0] = t0.x; v[u][k][1] = t0.y; v[u][k][2] = t0.z; v[u][k][3] = t0.w;
          v[u][k][4] = t1.x; v[u][k][5] = t1.y; v[u][k][6] = t1.z; v[u][k][7] = t1.w;
        } else if constexpr (DPL == 4) {
          const float4 t = *reinterpret_cast<const float4*>(src);
          v[u][k][0] = t.x; v[u][k][1] = t.y; v[u][k][2] = t.z; v[u][k][3] = t.w;
        } else {
          const float2 t = *reinterpret_cast<const float2*>(src);
          v[u][k][0] = t.x; v[u][k][1] = t.y;
        }
        M[u] = fmaxf(M[u], lse_v[u][k]);
      }
#pragma unroll
    for (int u = 0; u < RPI / 2; ++u) {
      float acc[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
      float wsum = 0.f;
      if (M[u] != kNegInf) {
#pragma unroll
        for (int k = 0; k < S; ++k) {
          // an empty run (lse -inf, and stale O) gets weight 0 by select
          const bool on = lse_v[u][k] != kNegInf;
          const float w = on ? fast_exp2((lse_v[u][k] - M[u]) * kLog2e) : 0.f;
          wsum += w;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, on ? v[u][k][e] : 0.f, acc[e]);
        }
      }
      const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] *= inv;
      if (!valid[u]) continue;
      const int64_t off = orow[u] * D + DPL * dl;
      if constexpr (DPL == 8) {
        if (p.out_f32) {
          float* o = reinterpret_cast<float*>(p.out) + off;
          *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
          *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        } else {
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + off) =
              make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        }
      } else if constexpr (DPL == 4) {
        if (p.out_f32)
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + off) =
              make_float4(acc[0], acc[1], acc[2], acc[3]);
        else
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + off) =
              make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      } else {
        if (p.out_f32)
          *reinterpret_cast<float2*>(reinterpret_cast<float*>(p.out) + off) =
              make_float2(acc[0], acc[1]);
        else
          *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.out) + off) =
              pack_bf16x2(acc[0], acc[1]);
      }
      if (p.lse && dl == 0)
        p.lse[orow[u]] = (M[u] == kNegInf) ? kNegInf : M[u] + fast_log2(wsum) * kLn2;
    }
  }
}

}  // namespace

template <int D>
hipError_t launch_tile_merge_d(const TileMergeParams& p, int nx, hipStream_t stream) {
  const dim3 grid((unsigned)(nx * p.num_kv_heads)), block(prefill_detail::kThreads);
  switch (p.tile_splits) {
    case 2: hipLaunchKernelGGL((tile_merge_kernel<2, D>), grid, block, 0, stream, p, nx); break;
    case 3: hipLaunchKernelGGL((tile_merge_kernel<3, D>), grid, block, 0, stream, p, nx); break;
    case 4: hipLaunchKernelGGL((tile_merge_kernel<4, D>), grid, block, 0, stream, p, nx); break;
    case 5: hipLaunchKernelGGL((tile_merge_kernel<5, D>), grid, block, 0, stream, p, nx); break;
    case 6: hipLaunchKernelGGL((tile_merge_kernel<6, D>), grid, block, 0, stream, p, nx); break;
    case 7: hipLaunchKernelGGL((tile_merge_kernel<7, D>), grid, block, 0, stream, p, nx); break;
    case 8: hipLaunchKernelGGL((tile_merge_kernel<8, D>), grid, block, 0, stream, p, nx); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tile_merge(const TileMergeParams& p, int nx, int head_dim, hipStream_t stream) {
  if (nx <= 0) return hipSuccess;
  if (head_dim == 64) return launch_tile_merge_d<64>(p, nx, stream);
  if (head_dim == kHeadDim) return launch_tile_merge_d<kHeadDim>(p, nx, stream);
  if (head_dim == 256) return launch_tile_merge_d<256>(p, nx, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_unit_merge(const ReduceParams& p, int units, int unit_rows,
                             hipStream_t stream) {
  if (units <= 0 || unit_rows <= 0) return hipSuccess;
  if ((int64_t)units * unit_rows >= kUnitMergeMinRows) {
    hipLaunchKernelGGL(unit_merge_kernel, dim3(units), dim3(kThreads), 0, stream, p);
  } else {
    ReduceParams q = p;
    q.unit_rows = unit_rows;
    hipLaunchKernelGGL(splitkv_reduce_kernel, dim3(units, unit_rows), dim3(kThreads), 0, stream,
                       q);
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(splitkv_reduce_kernel, dim3(p.rows), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
