// Device helpers shared by the gfx950 kernels: bf16 and MX decodes, wave
// reductions, and the workspace plan written by the routing kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 ----

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// dot of two packed bf16 pairs accumulated into fp32 (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// ------------------------------------------------------------------ MX ----

// E8M0 scale byte -> 2^(b-127) as fp32 (b <= 1 give subnormals); 255 -> NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b == 255u ? __uint_as_float(0x7FC00000u) : __builtin_ldexpf(1.0f, int(b) - 127);
}

// Byte SEL of a packed word of E2M1 codes -> two bf16 values (unscaled,
// exact: every E2M1 value is a bf16).  Low nibble -> element 0 (low half).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// Byte SEL of a packed word of E2M1 codes -> two fp32 values (unscaled).
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// ------------------------------------------------------------ reductions --

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// --------------------------------------------------------------- plan -----
// Token -> expert grouping written by the plan kernel and read by the expert
// kernels.  Pair p = t * top_k + j is slot j of token t.
struct Plan {
  int32_t* n_active;  // [1] number of experts with at least one pair
  int32_t* active;    // [E] expert ids with pairs, ascending
  int32_t* act_off;   // [E + 1] start of each active expert's pairs in `pairs`
  int32_t* pairs;     // [T * k] pair ids grouped by expert, ascending within
};

}  // namespace moe
