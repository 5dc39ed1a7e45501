// Paged GQA decode kernels (split-KV) for gfx950: thin wrappers around
// decode_body (pa_decode_body.h) with their own LDS, one workgroup per
// (split, kv head, sequence).
#include "pa_decode_body.h"

namespace pa {

namespace {

using decode_detail::decode_body;
using decode_detail::decode_smem_floats;

template <int G, int W, bool FUSED>
__global__ __launch_bounds__(64 * W) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float sm_buf[decode_smem_floats<G, W>()];
  decode_body<G, W, FUSED>(p, blockIdx.x, blockIdx.y, blockIdx.z, sm_buf);
}

template <int W, bool FUSED>
hipError_t launch_w(const DecodeParams& p, int group, dim3 grid, hipStream_t stream) {
  dim3 block(64 * W);
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_kernel<1, W, FUSED>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<2, W, FUSED>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<4, W, FUSED>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<8, W, FUSED>), grid, block, 0, stream, p); break;
    case 16:
      if constexpr (W == 4) {
        hipLaunchKernelGGL((decode_kernel<16, 4, FUSED>), grid, block, 0, stream, p);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int group, int waves, bool fused,
                         hipStream_t stream) {
  dim3 grid(p.num_splits, p.num_kv_heads, p.num_seqs);
  if (waves == 4) return fused ? launch_w<4, true>(p, group, grid, stream)
                               : launch_w<4, false>(p, group, grid, stream);
  if (waves == 8) return fused ? launch_w<8, true>(p, group, grid, stream)
                               : launch_w<8, false>(p, group, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
