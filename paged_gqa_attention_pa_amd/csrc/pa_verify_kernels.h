// Short-run kernel instantiations (included by the per-head-dim sources):
// one verify_kernel per (G, row blocks RB, precise P, head dim D), the even-work
// grid of the decode path driving verify_body (pa_verify_body.h).
#pragma once

#include "pa_even_grid.h"

namespace pa {
namespace verify_detail {

constexpr int kVerifyWaves = 4;

// Two workgroups per CU where the accumulators allow (at most two row blocks
// per wavefront, which four row blocks get by sharing a tile stream between
// two wavefronts, at D <= 128), so that two wavefronts per SIMD keep loads in
// flight; otherwise one, with the accumulators in AGPRs.
template <int RB, int D>
constexpr int verify_min_blocks() {
  return D <= 128 ? 2 : 1;
}

template <int G, int RB, bool PRECISE, int D>
__global__ __launch_bounds__(64 * kVerifyWaves, (verify_min_blocks<RB, D>())) void verify_kernel(
    DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float sm_buf[verify_smem_floats<kVerifyWaves, D>()];
  decode_detail::decode_even_body<G, kVerifyWaves, RB, PRECISE, D>(p, blockIdx.x, gridDim.x,
                                                                  sm_buf);
}

// Built: RB in {1, 2, 4} at D <= 128 and {1, 2} at D = 256 (16 rows x 256
// dims per block), and only where one token's G rows fit (G <= 16 * RB).
template <int G, int RB, bool PRECISE, int D>
const void* kernel_of() {
  if constexpr ((D > 128 && RB > 2) || G > 16 * RB) return nullptr;
  else return reinterpret_cast<const void*>(&verify_kernel<G, RB, PRECISE, D>);
}

template <int G, bool PRECISE, int D>
const void* by_row_blocks(int rb) {
  switch (rb) {
    case 1: return kernel_of<G, 1, PRECISE, D>();
    case 2: return kernel_of<G, 2, PRECISE, D>();
    case 4: return kernel_of<G, 4, PRECISE, D>();
    default: return nullptr;
  }
}

template <bool PRECISE, int D>
const void* by_group(int group, int rb) {
  switch (group) {
    case 1: return by_row_blocks<1, PRECISE, D>(rb);
    case 2: return by_row_blocks<2, PRECISE, D>(rb);
    case 4: return by_row_blocks<4, PRECISE, D>(rb);
    case 8: return by_row_blocks<8, PRECISE, D>(rb);
    case 16: return by_row_blocks<16, PRECISE, D>(rb);
    case 32: return by_row_blocks<32, PRECISE, D>(rb);
    default: return nullptr;
  }
}

// Defined in pa_verify_d64.hip, pa_verify_d128.hip, pa_verify_d256.hip.
const void* verify_ptr_d64(int group, int rb, bool precise);
const void* verify_ptr_d128(int group, int rb, bool precise);
const void* verify_ptr_d256(int group, int rb, bool precise);

}  // namespace verify_detail
}  // namespace pa
