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

namespace pa {

namespace {

constexpr int kThreads = 256;

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
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t orow = row;
  if (p.query_start_loc) {  // mixed batch: merge the single-token sequences only
    const int s = row / p.num_q_heads;
    const int q0 = p.query_start_loc[s];
    if (p.query_start_loc[s + 1] - q0 != 1) return;
    orow = (int64_t)q0 * p.num_q_heads + row % p.num_q_heads;
  }
  const int S = p.num_splits;
  const int D = p.head_dim;
  const float* lse_row = p.part_lse + (int64_t)row * S;

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

  const int items = D / 4;
  for (int base = 0; base < items; base += kThreads) {
    const int chunk = min(kThreads, items - base);
    const int groups = kThreads / chunk;
    const int item = base + tid % chunk;
    const int grp = tid / chunk;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (grp < groups && M != kNegInf) {
      const float* src = p.part_o + (int64_t)row * S * D + 4 * item;
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

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(splitkv_reduce_kernel, dim3(p.rows), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
