// Short-query-run kernels for gfx950 (speculative-decode verification
// batches: every sequence has 1 <= q_s query tokens with q_s * G <= 64; also
// decode at G = 32, one token of 32 heads being two 16-row blocks, and every
// decode or short run at head dims 64 and 256): the
// even-work grid of the decode path driving verify_body (pa_verify_body.h),
// one instantiation per (G, row blocks RB, precise P, head dim D).  Rows are
// (token, q head) pairs: partials are [T*Hq, slots, D].
#include <atomic>

#include "pa_even_grid.h"

namespace pa {

namespace {

using decode_detail::decode_even_body;
using verify_detail::verify_smem_floats;

constexpr int kVerifyWaves = 4;

// Two workgroups per CU where the accumulators allow (at most two row blocks
// per wavefront, which four row blocks get by pairing wavefronts, at
// D <= 128), so that two wavefronts per SIMD keep loads in flight; otherwise
// one, with the accumulators in AGPRs.
template <int RB, int D>
constexpr int verify_min_blocks() {
  return (RB <= 4 && D <= 128) ? 2 : 1;
}

template <int G, int RB, bool PRECISE, int D>
__global__ __launch_bounds__(64 * kVerifyWaves, (verify_min_blocks<RB, D>())) void verify_kernel(
    DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float sm_buf[verify_smem_floats<kVerifyWaves, D>()];
  decode_even_body<G, kVerifyWaves, RB, PRECISE, D>(p, blockIdx.x, gridDim.x, sm_buf);
}

// Four row blocks at D = 256 (256 accumulators per lane) are not built.
template <int G, int RB, bool PRECISE, int D>
const void* kernel_of() {
  if constexpr (RB * D > 512) return nullptr;
  else return reinterpret_cast<const void*>(&verify_kernel<G, RB, PRECISE, D>);
}

// Row blocks built per G: q_s * G <= 16 * RB, RB in {1, 2, 4} (G = 1: q_s <= 16
// is one block; G = 32: one or two tokens, two or four blocks).
template <bool PRECISE, int D>
const void* verify_ptr_pd(int group, int rb) {
  switch (group) {
    case 1: return rb == 1 ? kernel_of<1, 1, PRECISE, D>() : nullptr;
    case 2:
      return rb == 1 ? kernel_of<2, 1, PRECISE, D>() : rb == 2 ? kernel_of<2, 2, PRECISE, D>() : nullptr;
    case 4:
      return rb == 1   ? kernel_of<4, 1, PRECISE, D>()
             : rb == 2 ? kernel_of<4, 2, PRECISE, D>()
             : rb == 4 ? kernel_of<4, 4, PRECISE, D>()
                       : nullptr;
    case 8:
      return rb == 1   ? kernel_of<8, 1, PRECISE, D>()
             : rb == 2 ? kernel_of<8, 2, PRECISE, D>()
             : rb == 4 ? kernel_of<8, 4, PRECISE, D>()
                       : nullptr;
    case 16:
      return rb == 1   ? kernel_of<16, 1, PRECISE, D>()
             : rb == 2 ? kernel_of<16, 2, PRECISE, D>()
             : rb == 4 ? kernel_of<16, 4, PRECISE, D>()
                       : nullptr;
    case 32:
      return rb == 2 ? kernel_of<32, 2, PRECISE, D>() : rb == 4 ? kernel_of<32, 4, PRECISE, D>() : nullptr;
    default: return nullptr;
  }
}

template <int D>
const void* verify_ptr_d(int group, int rb, bool precise) {
  return precise ? verify_ptr_pd<true, D>(group, rb) : verify_ptr_pd<false, D>(group, rb);
}

const void* verify_ptr(int group, int rb, bool precise, int head_dim) {
  switch (head_dim) {
    case 64: return verify_ptr_d<64>(group, rb, precise);
    case 128: return verify_ptr_d<128>(group, rb, precise);
    case 256: return verify_ptr_d<256>(group, rb, precise);
    default: return nullptr;
  }
}

int rb_index(int rb) { return rb == 1 ? 0 : rb == 2 ? 1 : 2; }
int group_index(int g) {
  return g == 1 ? 0 : g == 2 ? 1 : g == 4 ? 2 : g == 8 ? 3 : g == 16 ? 4 : 5;
}
int dim_index(int d) { return d == 64 ? 0 : d == 128 ? 1 : 2; }

}  // namespace

int verify_row_blocks(int group, int max_query_len, int head_dim) {
  const int rows = group * max_query_len;
  const int rb = rows <= 16 ? 1 : rows <= 32 ? 2 : rows <= 64 ? 4 : 0;
  return rb * head_dim > 512 ? 0 : rb;
}

int verify_resident(int group, int rb, bool precise, int head_dim) {
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs][6][3][2][3];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 0;
  std::atomic<int>& slot =
      cache[dev][group_index(group)][rb_index(rb)][precise ? 1 : 0][dim_index(head_dim)];
  const int cached = slot.load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  const void* k = verify_ptr(group, rb, precise, head_dim);
  int cus = 0, per_cu = 0;
  if (!k || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64 * kVerifyWaves, 0) != hipSuccess)
    return 0;
  const int n = cus * (per_cu > 0 ? per_cu : 1);
  slot.store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_verify(const DecodeParams& p, int group, int rb, bool precise, int head_dim,
                         int nw, hipStream_t stream) {
  const void* k = verify_ptr(group, rb, precise, head_dim);
  if (!k || nw <= 0) return hipErrorInvalidValue;
  DecodeParams a = p;
  void* args[] = {&a};
  return hipLaunchKernel(k, dim3(nw), dim3(64 * kVerifyWaves), args, 0, stream);
}

}  // namespace pa
