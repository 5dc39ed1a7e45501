// Short-query-run launches for gfx950 (speculative-decode verification
// batches: every sequence has 1 <= q_s query tokens with q_s * G <= 64, 32
// at head dim 256; also decode at G = 32, one token of 32 heads being two
// 16-row blocks, and every decode at head dims 64 and 256): kernel lookup,
// occupancy and launch of the instantiations in pa_verify_d*.hip.  Rows are
// (token, q head) pairs: partials are [T*Hq, slots, D].
#include <atomic>

#include "pa_verify_kernels.h"

namespace pa {

namespace {

using verify_detail::kVerifyWaves;

const void* verify_ptr(int group, int rb, bool precise, int head_dim) {
  switch (head_dim) {
    case 64: return verify_detail::verify_ptr_d64(group, rb, precise);
    case 128: return verify_detail::verify_ptr_d128(group, rb, precise);
    case 256: return verify_detail::verify_ptr_d256(group, rb, precise);
    default: return nullptr;
  }
}

int rb_index(int rb) { return rb == 1 ? 0 : rb == 2 ? 1 : rb == 4 ? 2 : 3; }
int group_index(int g) {
  return g == 1 ? 0 : g == 2 ? 1 : g == 4 ? 2 : g == 8 ? 3 : g == 16 ? 4 : 5;
}
int dim_index(int d) { return d == 64 ? 0 : d == 128 ? 1 : 2; }

}  // namespace

// Eight row blocks (128 rows, four wavefronts on one tile stream) measured
// no faster than the query tiles on gfx950 (64 sequences, contexts
// U[128, 8192]: G = 8, q = 16: 470 us against 446 us; G = 16, q = 8: 468
// against 462), so runs above 64 rows take the query tiles.
int verify_row_blocks(int group, int max_query_len, int head_dim) {
  const int rows = group * max_query_len;
  const int rb = rows <= 16 ? 1 : rows <= 32 ? 2 : rows <= 64 ? 4 : 0;
  return (head_dim > 128 && rb > 2) ? 0 : rb;
}

int verify_resident(int group, int rb, bool precise, int head_dim, hipStream_t stream) {
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs][6][4][2][3];
  const int dev = stream_device(stream);
  if (dev < 0 || dev >= kDevs) return 0;
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
