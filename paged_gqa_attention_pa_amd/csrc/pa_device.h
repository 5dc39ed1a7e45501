// Device helpers shared by the gfx950 kernels: bf16 packing, MFMA operand
// types, wavefront broadcasts and reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// One 16-byte global load (global_load_dwordx4).
__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// bf16 pair packed in a dword -> two floats (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Sum of a packed bf16 pair added to acc in fp32 (v_dot2c_f32_bf16 with
// weights 1, 1): the pair's values are exact in fp32.
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of `v` held by lane (lane & ~(W-1)) + k, for W in {1, 2, 4}: a DPP
// quad_perm broadcast inside each group of four lanes.
template <int K>
__device__ __forceinline__ float quad_bcast(float v) {
  constexpr int ctrl = K | (K << 2) | (K << 4) | (K << 6);
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xf, 0xf, false));
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, 64); }

__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

// Lanes l and l ^ 32 exchange v (v_permlane32_swap, no LDS round trip).
// Returns {value of the lane in the lower half, value of the lane in the
// upper half} of the pair, the same on both lanes.
__device__ __forceinline__ f32x2 halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return (f32x2){__uint_as_float(r[0]), __uint_as_float(r[1])};
}

}  // namespace pa
