// Prefill path: the routed experts as grouped GEMMs on gfx950's block-scaled
// matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4), MXFP4 weights times
// MXFP8 activations, fp32 accumulation.
//
// Deltafin explainer (bhfrc.com), section 2.1: prefill runs the experts with
// MXFP8 activations against the MXFP4 weights; section 6.2: the weights are
// consumed in their quantised form inside the product.  Here both operands
// stay in their MX encodings all the way into the matrix core, which
// applies the E8M0 block exponents itself.
//
// Operand layout of the instruction with A = FP4 (cbsz 4) and B = FP8 E4M3
// (blgp 0), established on gfx950 with one-hot and exact-arithmetic probes
// (wave64, lane l: g = l / 16, c = l % 16; K below is the position in the
// 128-wide tile with MX blocks contiguous, block q = K / 32):
//   A lane (c, g): 16 bytes = elements K = 32 g .. 32 g + 31 of row c, low
//     nibble first -- exactly lane l of a packed weight tile (pack.hip);
//   B lane (c, g): bytes 0..15 = K = 16 g .. 16 g + 15 and bytes 16..31 =
//     K = 64 + 16 g .. 64 + 16 g + 15 of column c;
//   scales: block q of row (column) c is scaled by byte `opsel` of the
//     scale operand of lane 16 q + c, for A and B alike;
//   D: lane l holds rows 4 g .. 4 g + 3 of column c.
// A 4-tile super-step of the packed weights keeps a lane's four tile
// exponents in one dword, so tile j of the step uses opsel j.  The staged
// activations keep the same convention: per token and super-step, 16 scale
// bytes ordered [g][j] (block 16 kq + 4 j + g at byte 4 g + j), so lane g's
// dword holds its four tiles' exponents.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace mx {

constexpr int kTok = kPlanTileTokens;  // tokens (B columns) per tile, 4 MFMA column groups
constexpr int kSub = kTok / 16;
constexpr int kStep = 512;             // contraction columns per super-step (4 tiles)
constexpr int kRowB = kStep + 16;      // staged bytes per token and step: codes + 16 scale bytes
constexpr int kStageBytes = kTok * kRowB;  // 33 KiB: 33 wave-wide 1 KiB loads
constexpr int kNS = 4;                 // A streams (16-row groups x matrices) per wave

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// Position of the scale byte of block b (along the contraction) in the
// MFMA-ordered scale row (see the header comment).
__host__ __device__ __forceinline__ int scale_pos(int b) {
  return (b & ~15) | ((b & 3) << 2) | ((b & 15) >> 2);
}

template <int J>
__device__ __forceinline__ f32x4 mma(u32x4 a, i32x8 b, f32x4 c, uint32_t sa, uint32_t sb) {
  const i32x8 av = {int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, c, 4, 0, J, int(sa), J,
                                                          int(sb));
}

// One super-step of A operands for a wave: kNS streams x 4 tiles + the
// streams' exponent dwords.
struct ATiles {
  u32x4 w[kNS][4];
  uint32_t s[kNS];
};

// Streams of a wave: code tiles of a 16-row group (base + 16 lane) and the
// lane's exponent bytes (nkb4 per lane, tile kb at byte kb).
struct AStreams {
  const uint8_t* codes[kNS];
  const uint8_t* scl[kNS];
  int nkb;
};

__device__ __forceinline__ void load_a(ATiles& t, const AStreams& st, int kq) {
#pragma unroll
  for (int s = 0; s < kNS; ++s) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t.w[s][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          st.codes[s] + size_t(min(4 * kq + j, st.nkb - 1)) * 1024));
    t.s[s] = *reinterpret_cast<const uint32_t*>(st.scl[s] + 4 * kq);
  }
}

// Issues the wave's share of one super-step of activations straight into
// LDS (no registers): 33 wave-wide 16-byte-per-lane loads fill kTok token
// rows of kRowB bytes; wave w issues loads w, w + 4, ...  row(j) gives
// token j's code row (kStep bytes of this step at +kq * kStep) and srow(j)
// its MFMA-ordered scale row (16 bytes of this step at +kq * 16).
template <typename Row, typename SRow>
__device__ __forceinline__ void stage_b(uint8_t* lds, int kq, Row row, SRow srow) {
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int lane = threadIdx.x % kWave;
  for (int n = wave; n < kStageBytes / 1024; n += 4) {
    const int chunk = n * 64 + lane;  // 16-byte chunk of the staged block
    const int j = chunk / (kRowB / 16), q = chunk % (kRowB / 16);
    const uint8_t* src = q < kStep / 16 ? row(j) + size_t(kq) * kStep + 16 * q
                                        : srow(j) + size_t(kq) * 16;
    __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)(lds + n * 1024), 16, 0, 0);
  }
}

// acc[s][u] += A stream s (this step's 4 tiles) x B columns 16 u .. 16 u + 15.
__device__ __forceinline__ void mma_step(f32x4 (&acc)[kNS][kSub], const ATiles& a,
                                         const uint8_t* lds) {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    const uint8_t* r = lds + (16 * u + c) * kRowB;
    const uint32_t sb = *reinterpret_cast<const uint32_t*>(r + kStep + 4 * g);
#define MX_TILE(J)                                                                        \
  {                                                                                      \
    const u32x4 lo = *reinterpret_cast<const u32x4*>(r + 128 * J + 16 * g);             \
    const u32x4 hi = *reinterpret_cast<const u32x4*>(r + 128 * J + 64 + 16 * g);        \
    const i32x8 b = {int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),                     \
                     int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};                    \
    _Pragma("unroll") for (int s = 0; s < kNS; ++s) acc[s][u] =                          \
        mma<J>(a.w[s][J], b, acc[s][u], a.s[s], sb);                                     \
  }
    MX_TILE(0)
    MX_TILE(1)
    MX_TILE(2)
    MX_TILE(3)
#undef MX_TILE
  }
}

// The contraction of one tile: nkq super-steps, A double-buffered in
// registers, B double-buffered in LDS (two kStageBytes buffers at lds).
// All threads of the workgroup must call it.
template <typename Row, typename SRow>
__device__ __forceinline__ void gemm_tile(f32x4 (&acc)[kNS][kSub], const AStreams& st, int nkq,
                                          uint8_t* lds, Row row, SRow srow) {
#pragma unroll
  for (int s = 0; s < kNS; ++s)
#pragma unroll
    for (int u = 0; u < kSub; ++u) acc[s][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  ATiles ta, tb;
  stage_b(lds, 0, row, srow);
  load_a(ta, st, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto step = [&](ATiles& cur, ATiles& nxt, int kq) {
    // loads of step kq + 1: activations into the other LDS buffer, weights
    // into the other registers; both in flight while step kq computes
    uint8_t* cur_l = lds + (kq & 1) * kStageBytes;
    uint8_t* nxt_l = lds + ((kq + 1) & 1) * kStageBytes;
    stage_b(nxt_l, kq + 1, row, srow);
    load_a(nxt, st, kq + 1);
    mma_step(acc, cur, cur_l);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int kq = 0;
  for (; kq + 2 < nkq; kq += 2) {
    step(ta, tb, kq);
    step(tb, ta, kq + 1);
  }
  if (kq + 1 < nkq) {
    step(ta, tb, kq);
    mma_step(acc, tb, lds + ((kq + 1) & 1) * kStageBytes);
  } else {
    mma_step(acc, ta, lds + (kq & 1) * kStageBytes);
  }
}

}  // namespace mx
}  // namespace moe
