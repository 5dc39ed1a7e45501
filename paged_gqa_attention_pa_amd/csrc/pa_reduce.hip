// Log-sum-exp merge of split-KV partials (the exact merge behind the
// parallel tiled softmax of the IBM Triton summary's five-step list; the
// algebra is that of the online-softmax statistics m and l, guide section
// "Flash Attention革命"):
//   M = max_k lse_k, w_k = exp(lse_k - M),
//   O = sum_k w_k O_k / sum_k w_k,  LSE = M + ln sum_k w_k,
// and O = 0, LSE = -inf when every split is empty.  Empty splits (lse = -inf)
// get weight 0 without evaluating -inf - (-inf).
//
// One wavefront per row; lane i owns dims 4i..4i+3 (float4 loads and
// stores), looping when head_dim > 256.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

__global__ __launch_bounds__(64) void splitkv_reduce_kernel(ReduceParams p) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const int S = p.num_splits;
  const int D = p.head_dim;
  const float* lse_row = p.part_lse + (int64_t)row * S;

  float M = kNegInf;
  for (int k = lane; k < S; k += 64) M = fmaxf(M, lse_row[k]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));

  float wsum = 0.f;
  if (M != kNegInf) {
    for (int k = lane; k < S; k += 64) {
      const float lk = lse_row[k];
      if (lk != kNegInf) wsum += fast_exp2((lk - M) * kLog2e);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wsum += shfl_xor(wsum, off);
  }
  const float inv = (M != kNegInf) ? 1.f / wsum : 0.f;

  for (int d0 = 4 * lane; d0 < D; d0 += 256) {
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != kNegInf) {
      for (int k = 0; k < S; ++k) {
        const float lk = lse_row[k];
        if (lk == kNegInf) continue;
        const float w = fast_exp2((lk - M) * kLog2e);
        const float4 ok = *reinterpret_cast<const float4*>(p.part_o + ((int64_t)row * S + k) * D + d0);
        o.x = fmaf(w, ok.x, o.x);
        o.y = fmaf(w, ok.y, o.y);
        o.z = fmaf(w, ok.z, o.z);
        o.w = fmaf(w, ok.w, o.w);
      }
      o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
    }
    if (p.out_f32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + (int64_t)row * D + d0) = o;
    } else {
      uint2 packed = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + (int64_t)row * D + d0) = packed;
    }
  }
  if (p.lse && lane == 0) p.lse[row] = (M == kNegInf) ? kNegInf : M + fast_log2(wsum) * kLn2;
}

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(splitkv_reduce_kernel, dim3(p.rows), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
