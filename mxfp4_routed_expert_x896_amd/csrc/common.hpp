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

// Eight E2M1 codes (one dword, low nibble first) times the fp32 scale sc,
// as eight bf16 (v_cvt_scalef32_pk_bf16_fp4).  For sc = 2^e this is exact:
// every E2M1 value times a power of two is a bf16 (subnormals included) up
// to overflow; a NaN scale gives NaN.
__device__ __forceinline__ u32x4 fp4x8_scaled(uint32_t w, float sc) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  return r;
}

// ------------------------------------------------------------ reductions --
// Wave-wide reductions with DPP row operations (a few cycles per step, no
// LDS round trip): quad swaps, half-row and row mirrors, then the row
// broadcasts; the total ends in lane 63 and is broadcast with readlane.

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xF, false));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_sum_step(float v) {
  return v + __uint_as_float(dpp_or_zero<CTRL, ROW_MASK>(__float_as_uint(v)));
}

// Sum over all 64 lanes (every lane must be active); result in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_sum_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_sum_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_sum_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_sum_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_sum_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_sum_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(__float_as_uint(v)), 63)));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const uint64_t o = (uint64_t(dpp_or_zero<CTRL, ROW_MASK>(uint32_t(v >> 32))) << 32) |
                     dpp_or_zero<CTRL, ROW_MASK>(uint32_t(v));
  return o > v ? o : v;
}

// Maximum of an unsigned 64-bit key over all 64 lanes; result in every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);
  v = dpp_max_step<0x4E, 0xF>(v);
  v = dpp_max_step<0x141, 0xF>(v);
  v = dpp_max_step<0x140, 0xF>(v);
  v = dpp_max_step<0x142, 0xA>(v);
  v = dpp_max_step<0x143, 0xC>(v);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), 63));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), 63));
  return (uint64_t(hi) << 32) | lo;
}

// ------------------------------------------------------------- layout -----
// MFMA-tiled MXFP4 matrix (written by the pack kernels, see pack.hip): code
// tiles of 16 rows x 128 columns (1 KiB, lane order), then the scales: per
// row group and super-step (4 tiles), 64 lane dwords (256 contiguous bytes),
// lane l's dword holding its four tiles' exponents.
struct PackedMx {
  int nb, nkb, nkb4;   // blocks per row, 128-column tiles per row group, nkb rounded to 4
  int nsup;            // super-steps per row group (nkb4 / 4)
  size_t code_bytes;   // offset of the scales
  size_t bytes;        // whole matrix
  __host__ __device__ PackedMx(int R, int K) {
    nb = K / 32;
    nkb = (nb + 3) / 4;
    nkb4 = (nkb + 3) / 4 * 4;
    nsup = nkb4 / 4;
    code_bytes = size_t(R / 16) * nkb * 1024;
    bytes = code_bytes + size_t(R / 16) * 64 * nkb4;
  }
  // byte offset of lane l's exponent dword of super-step q of row group rg
  __host__ __device__ size_t scale_dword(int rg, int q, int l) const {
    return code_bytes + ((size_t(rg) * nsup + q) * 64 + l) * 4;
  }
};

// --------------------------------------------------------------- plan -----
// Token -> expert grouping written by the plan builder (plan.hpp) and read
// by the expert kernels.  Pair p = t * top_k + j is slot j of token t.
struct Plan {
  int32_t* n_active;  // [1] number of experts with at least one pair
  int32_t* active;    // [E] expert ids with pairs, ascending
  int32_t* act_off;   // [E + 1] start of each active expert's pairs in `pairs`
  int32_t* pairs;     // [T * k] pair ids grouped by expert
  int32_t* n_mtiles;  // [1] number of token tiles (kPlanTileTokens pairs of one expert)
  int32_t* mtiles;    // [<= E + T * k / kPlanTileTokens] slot << 16 | tile index within the slot
};

// Pairs per token tile of the prefill (MFMA) path.
constexpr int kPlanTileTokens = 96;

// floor(log2 |a|) of a non-zero finite fp32 (normal or subnormal).
__device__ __forceinline__ int floor_log2_f32(float a) {
  const uint32_t u = __float_as_uint(a) & 0x7FFFFFFFu;
  const int f = int(u >> 23);
  if (f > 0) return f - 127;
  return (31 - __clz(int(u))) - 149;
}

// E4M3FN code of v (finite), round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal step 2^-9
    const uint32_t q = uint32_t(rintf(a * 512.0f));  // 0..8; 8 is the first normal
    return sign | q;
  }
  int e = floor_log2_f32(a);  // -6 .. 8
  uint32_t q = uint32_t(rintf(__builtin_ldexpf(a, 3 - e)));  // 8 .. 16
  if (q == 16u) {
    q = 8u;
    e += 1;
  }
  return sign | (uint32_t(e + 7) << 3) | (q - 8u);
}

// MXFP8 block exponent for a block with largest magnitude amax (OCP MX
// rule as read here): clamp(floor(log2 amax) - 8, -127, 127), -127 for 0.
__device__ __forceinline__ int mxfp8_block_exp(float amax) {
  const int E = amax == 0.0f ? -127 : floor_log2_f32(amax) - 8;
  return max(-127, min(127, E));
}

// E2M1 code (0..15, sign in bit 3) of v, round to nearest even, saturating
// at +-6.  The magnitude grid has step 0.5 below 2, 1 below 4 and 2 up to 6;
// rintf (round half to even under the default mode) picks the even multiple
// of the step, which is the code with its mantissa bit clear, and a tie at a
// binade's top rounds up onto the next binade's even code (1.75 -> 2).
__device__ __forceinline__ uint32_t e2m1_rne_sat(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  const float a = fminf(fabsf(v), 6.0f);
  float q;
  if (a < 2.0f) q = rintf(a * 2.0f) * 0.5f;
  else if (a < 4.0f) q = rintf(a);
  else q = rintf(a * 0.5f) * 2.0f;
  // magnitudes 0, 0.5, 1, 1.5 -> codes 0..3; 2, 3 -> 4, 5; 4 -> 6; 6 -> 7
  const uint32_t code = q < 2.0f ? uint32_t(q * 2.0f) : q < 4.0f ? uint32_t(q) + 2u
                                                        : q < 5.0f ? 6u : 7u;
  return sign | code;
}

// MXFP4 block exponent (the MXFP8 rule with E2M1's largest normal exponent,
// 2): clamp(floor(log2 amax) - 2, -127, 127), -127 for 0.
__device__ __forceinline__ int mxfp4_block_exp(float amax) {
  const int E = amax == 0.0f ? -127 : floor_log2_f32(amax) - 2;
  return max(-127, min(127, E));
}

// Results that cross workgroups of one launch (and XCDs, whose L2s are
// private) are stored and re-read with device-scope atomic accesses, which
// the compiler emits as write-through stores and L2-bypassing loads, instead
// of fencing (a device-scope fence writes back and invalidates the whole L2).
template <typename V>
__device__ __forceinline__ void store_coherent(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V load_coherent(const V* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe
