// Paged GQA decode kernels (split-KV) for gfx950: thin wrappers around
// decode_body (pa_decode_body.h) with their own LDS: the static grid, one
// workgroup per (split, kv head, sequence), and the even-work grid, a fixed
// number of workgroups sharing all tiles equally (decode_even_body).
#include <atomic>

#include "pa_even_grid.h"

namespace pa {

namespace {

using decode_detail::decode_body;
using decode_detail::decode_even_body;
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
    case 16: hipLaunchKernelGGL((decode_kernel<16, W, FUSED>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int G, int W>
__global__ __launch_bounds__(64 * W) void decode_even_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float sm_buf[decode_smem_floats<G, W>()];
  decode_even_body<G, W>(p, blockIdx.x, gridDim.x, sm_buf);
}

template <int W>
const void* even_kernel_ptr(int group) {
  switch (group) {
    case 1: return reinterpret_cast<const void*>(&decode_even_kernel<1, W>);
    case 2: return reinterpret_cast<const void*>(&decode_even_kernel<2, W>);
    case 4: return reinterpret_cast<const void*>(&decode_even_kernel<4, W>);
    case 8: return reinterpret_cast<const void*>(&decode_even_kernel<8, W>);
    case 16: return reinterpret_cast<const void*>(&decode_even_kernel<16, W>);
    default: return nullptr;
  }
}

const void* even_kernel(int group, int waves) {
  return waves == 4 ? even_kernel_ptr<4>(group) : waves == 8 ? even_kernel_ptr<8>(group) : nullptr;
}

}  // namespace

int stream_device(hipStream_t stream) {
  hipDevice_t dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return -1;
  return (int)dev;
}

int decode_even_resident(int group, int waves, hipStream_t stream) {
  // per device and (group, waves): CUs x resident workgroups per CU
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs][5][2];
  const int dev = stream_device(stream);
  if (dev < 0 || dev >= kDevs) return 0;
  const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : group == 8 ? 3 : 4;
  const int wi = waves == 8 ? 1 : 0;
  const int cached = cache[dev][gi][wi].load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  const void* k = even_kernel(group, waves);
  int cus = 0, per_cu = 0;
  if (!k || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64 * waves, 0) != hipSuccess)
    return 0;
  const int n = cus * (per_cu > 0 ? per_cu : 1);
  cache[dev][gi][wi].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_decode_even(const DecodeParams& p, int group, int waves, int nw,
                              hipStream_t stream) {
  const void* k = even_kernel(group, waves);
  if (!k || nw <= 0) return hipErrorInvalidValue;
  DecodeParams a = p;
  void* args[] = {&a};
  return hipLaunchKernel(k, dim3(nw), dim3(64 * waves), args, 0, stream);
}

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
