// The pa_prefill launch for gfx950: one kernel whose grid holds the
// prefill query tiles (prefill_body, pa_prefill_body.h) and, when the batch
// may contain single-token (decode) sequences, split-KV decode workgroups for
// them (decode_body, pa_decode_body.h), so a mixed serving batch is one
// launch (plus the LSE merge of the decode rows' splits).  Workgroup ids
// [0, nx*tile_splits*Hkv) are prefill tiles, the rest (split, kv head, sequence) decode
// work; both share one LDS buffer.  With tile_splits > 1 the tiles write
// partials, merged afterwards by tile_merge_kernel (pa_reduce.hip).
#include <atomic>

#include "pa_even_grid.h"
#include "pa_prefill_body.h"

namespace pa {

namespace {

using decode_detail::decode_body;
using decode_detail::decode_even_body;
using decode_detail::decode_smem_floats;
using prefill_detail::prefill_smem_bytes;
using prefill_detail::kThreads;
using prefill_detail::prefill_body;

constexpr int kDecodeWaves = kThreads / 64;

// Decode workgroups run with all kThreads threads; G = 16 and 32 are not
// built that way, nor head dims other than 128, so for those every sequence
// takes the prefill tiles.
template <int G, int D>
constexpr bool decode_part_built() {
  return D == kHeadDim && G * kDecodeWaves <= 64;
}

template <int G, int D>
constexpr int unified_smem_bytes() {
  if constexpr (decode_part_built<G, D>()) {
    return prefill_smem_bytes<D>() > decode_smem_floats<G, kDecodeWaves>() * 4
               ? prefill_smem_bytes<D>()
               : decode_smem_floats<G, kDecodeWaves>() * 4;
  } else {
    return prefill_smem_bytes<D>();
  }
}

template <int G, bool PRECISE, int D>
__global__ __launch_bounds__(kThreads, 2) void unified_kernel(PrefillParams pp, DecodeParams dp,
                                                              int nx) {
  __shared__ __attribute__((aligned(16))) char smem[unified_smem_bytes<G, D>()];
  const int n_pre = nx * pp.num_kv_heads * pp.tile_splits;
  const int id = blockIdx.x;
  if (id < n_pre) {
    prefill_body<G, PRECISE, D>(pp, id, nx, smem);
  } else if constexpr (decode_part_built<G, D>()) {
    const int d = id - n_pre;
    if (dp.piece_counts) {  // even-work grid over the single-token sequences
      decode_even_body<G, kDecodeWaves>(dp, d, gridDim.x - n_pre, reinterpret_cast<float*>(smem));
    } else {
      const int split = d % dp.num_splits;
      const int g = (d / dp.num_splits) % dp.num_kv_heads;
      const int b = d / (dp.num_splits * dp.num_kv_heads);
      decode_body<G, kDecodeWaves, false>(dp, split, g, b, reinterpret_cast<float*>(smem));
    }
  }
}

// Head dim 256: query tiles only (single-token sequences take the tiles
// too), four wavefronts with the whole register file of their SIMD.
template <int G, bool PRECISE>
__global__ __launch_bounds__(64 * prefill_detail::waves_of<256>(), 1) void prefill256_kernel(
    PrefillParams pp, DecodeParams dp, int nx) {
  __shared__ __attribute__((aligned(16))) char smem[prefill_smem_bytes<256>()];
  (void)dp;
  prefill_body<G, PRECISE, 256>(pp, blockIdx.x, nx, smem);
}

template <bool PRECISE>
const void* prefill256_ptr(int group) {
  switch (group) {
    case 1: return reinterpret_cast<const void*>(&prefill256_kernel<1, PRECISE>);
    case 2: return reinterpret_cast<const void*>(&prefill256_kernel<2, PRECISE>);
    case 4: return reinterpret_cast<const void*>(&prefill256_kernel<4, PRECISE>);
    case 8: return reinterpret_cast<const void*>(&prefill256_kernel<8, PRECISE>);
    case 16: return reinterpret_cast<const void*>(&prefill256_kernel<16, PRECISE>);
    case 32: return reinterpret_cast<const void*>(&prefill256_kernel<32, PRECISE>);
    default: return nullptr;
  }
}

template <bool PRECISE, int D>
const void* unified_ptr(int group) {
  switch (group) {
    case 1: return reinterpret_cast<const void*>(&unified_kernel<1, PRECISE, D>);
    case 2: return reinterpret_cast<const void*>(&unified_kernel<2, PRECISE, D>);
    case 4: return reinterpret_cast<const void*>(&unified_kernel<4, PRECISE, D>);
    case 8: return reinterpret_cast<const void*>(&unified_kernel<8, PRECISE, D>);
    case 16: return reinterpret_cast<const void*>(&unified_kernel<16, PRECISE, D>);
    case 32: return reinterpret_cast<const void*>(&unified_kernel<32, PRECISE, D>);
    default: return nullptr;
  }
}

const void* unified_kernel_of(int group, bool precise, int head_dim) {
  if (head_dim == 64) return precise ? unified_ptr<true, 64>(group) : unified_ptr<false, 64>(group);
  if (head_dim == kHeadDim)
    return precise ? unified_ptr<true, kHeadDim>(group) : unified_ptr<false, kHeadDim>(group);
  if (head_dim == 256) return precise ? prefill256_ptr<true>(group) : prefill256_ptr<false>(group);
  return nullptr;
}

}  // namespace

int unified_resident(int group, bool precise_p, int head_dim, hipStream_t stream) {
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs][6][2][2];
  const int dev = stream_device(stream);
  if (dev < 0 || dev >= kDevs) return 0;
  const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : group == 8 ? 3 : group == 16 ? 4 : 5;
  std::atomic<int>& slot = cache[dev][gi][precise_p ? 1 : 0][head_dim == 64 ? 0 : 1];
  const int cached = slot.load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  const void* k = unified_kernel_of(group, precise_p, head_dim);
  int cus = 0, per_cu = 0;
  if (!k || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, 0) != hipSuccess)
    return 0;
  const int n = cus * (per_cu > 0 ? per_cu : 1);
  slot.store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_prefill(const PrefillParams& pp, const DecodeParams& dp, int group, int nx,
                          int n_dec, bool precise_p, int head_dim, hipStream_t stream) {
  if ((int64_t)nx * pp.num_kv_heads + n_dec <= 0) return hipSuccess;
  if ((int64_t)nx * pp.num_kv_heads * pp.tile_splits + n_dec > 0x7fffffff)
    return hipErrorInvalidValue;
  const void* k = unified_kernel_of(group, precise_p, head_dim);
  if (!k) return hipErrorInvalidValue;
  // decode workgroups exist only where the kernel holds the decode part
  if (n_dec != 0 && !(head_dim == kHeadDim && group * kDecodeWaves <= 64))
    return hipErrorInvalidValue;
  PrefillParams a = pp;
  DecodeParams b = dp;
  int c = nx;
  void* args[] = {&a, &b, &c};
  const unsigned grid = (unsigned)((int64_t)nx * pp.num_kv_heads * pp.tile_splits + n_dec);
  const unsigned block = head_dim == 256 ? 64 * prefill_detail::waves_of<256>() : kThreads;
  return hipLaunchKernel(k, dim3(grid), dim3(block), args, 0, stream);
}

}  // namespace pa
