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
constexpr int kStageBytes = kTok * kStep;  // 32 KiB of activation codes per staging buffer (FP8)
constexpr int kNS = 4;                 // A streams (16-row groups x matrices) per wave

// B (activation) formats: the MFMA's blgp operand code.
constexpr int kFmtFp8 = 0;  // MXFP8: E4M3 codes, one byte per element
constexpr int kFmtFp4 = 4;  // MXFP4: E2M1 codes, two per byte, even element in the low nibble
// Bytes of one token's codes in one super-step, and of a staging buffer.
template <int BF>
constexpr int row_bytes() { return BF == kFmtFp4 ? kStep / 2 : kStep; }
template <int BF>
constexpr int stage_bytes() { return kTok * row_bytes<BF>(); }

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// s_waitcnt vmcnt(16) with expcnt and lgkmcnt left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kVmcnt16 = (1 << 14) | (7 << 4) | (15 << 8);
static_assert(kNS * 4 >= 16, "a step issues at least 16 ordinary loads after its staging");

// Position of the scale byte of block b (along the contraction) in the
// MFMA-ordered scale row (see the header comment).
__host__ __device__ __forceinline__ int scale_pos(int b) {
  return (b & ~15) | ((b & 3) << 2) | ((b & 15) >> 2);
}

template <int J, int BF>
__device__ __forceinline__ f32x4 mma(u32x4 a, i32x8 b, f32x4 c, uint32_t sa, uint32_t sb) {
  const i32x8 av = {int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, c, 4, BF, J, int(sa), J,
                                                          int(sb));
}

// One super-step of A operands for a wave: kNS streams x 4 tiles + the
// streams' exponent dwords.
struct ATiles {
  u32x4 w[kNS][4];
  uint32_t s[kNS];
};

// Streams of a wave: code tiles of a 16-row group and the lane's exponent
// bytes (nkb4 per lane, tile kb at byte kb).  The stream bases are uniform
// across the wave; the lane's part is a 32-bit offset shared by all streams
// (16 lane into a code tile, lane nkb4 into the exponents).
struct AStreams {
  const uint8_t* codes[kNS];
  const uint8_t* scl[kNS];
  uint32_t lane_code, lane_scl;
  int nkb;
};

__device__ __forceinline__ void load_a(ATiles& t, const AStreams& st, int kq) {
#pragma unroll
  for (int s = 0; s < kNS; ++s) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t.w[s][j] = *(reinterpret_cast<const u32x4*>(
          st.codes[s] + size_t(min(4 * kq + j, st.nkb - 1)) * 1024 + st.lane_code));
    t.s[s] = *reinterpret_cast<const uint32_t*>(st.scl[s] + 4 * kq + st.lane_scl);
  }
}

// Staged activations: token j's code bytes of a super-step (row_bytes: 512
// for FP8, 256 for FP4) as 16-byte chunks, chunk q at slot q ^ (j % 16) of
// the token's LDS row.  The 16 lanes that read the same chunk of 16
// consecutive tokens then hit 16 different bank groups, and a wave-wide
// staging load still fills 1 KiB of LDS contiguously (two FP8 token rows,
// four FP4 ones).
//
// Per lane, as 32-bit byte offsets from the wave-uniform bases: the global
// chunk each of the wave's staging loads fetches at super-step 0 (wave w
// issues loads w, w + 4, ..., covering the first 16 NSub tokens; 2 NSub
// loads for FP8, NSub for FP4), and the B exponent dword of each of its
// token groups.
template <int BF>
constexpr int tokens_per_load() { return 1024 / row_bytes<BF>(); }
template <int NSub, int BF>
constexpr int staging_loads() { return 16 * NSub / 4 / tokens_per_load<BF>(); }

template <int NSub, int BF>
struct BStage {
  const uint8_t* cbase;
  const uint8_t* sbase;
  uint32_t src[staging_loads<NSub, BF>()];
  uint32_t scl[NSub];
};

// row(j): token j's code row as a byte offset from cbase; srow(j): its
// MFMA-ordered exponent row as a byte offset from sbase.
template <int NSub, int BF, typename Row, typename SRow>
__device__ __forceinline__ void prepare_b(BStage<NSub, BF>& bs, const uint8_t* cbase,
                                          const uint8_t* sbase, Row row, SRow srow) {
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  constexpr int kChunks = row_bytes<BF>() / 16;  // chunks per token row: 32 (FP8), 16 (FP4)
  bs.cbase = cbase;
  bs.sbase = sbase;
#pragma unroll
  for (int i = 0; i < staging_loads<NSub, BF>(); ++i) {
    // token of this lane's LDS chunk, and the chunk whose slot the lane fills
    const int j = tokens_per_load<BF>() * (wave + 4 * i) + lane / kChunks;
    bs.src[i] = row(j) + 16 * ((lane % kChunks) ^ (j % 16));
  }
#pragma unroll
  for (int u = 0; u < NSub; ++u) bs.scl[u] = srow(16 * u + c) + 4 * g;
}

// One wave-wide 16-byte-per-lane load from global memory (base + lane's
// off) straight into LDS (lane l's bytes land at lds_addr + 16 l).  Issued
// as inline assembly so that the compiler's wait-count bookkeeping, which
// cannot order such loads against ordinary loads and would then wait for
// every load before the next MFMA, does not see it: the caller waits for it
// explicitly.  s_nop: one wait state between writing M0 and a load that
// reads it.
__device__ __forceinline__ void load_to_lds16(const uint8_t* base, uint32_t off,
                                              uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

template <int NSub, int BF>
__device__ __forceinline__ void stage_b(uint8_t* lds, int kq, const BStage<NSub, BF>& bs) {
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const uint8_t* base = bs.cbase + size_t(kq) * row_bytes<BF>();
  const uint32_t l0 = uint32_t(reinterpret_cast<uintptr_t>((lvoid*)lds));
#pragma unroll
  for (int i = 0; i < staging_loads<NSub, BF>(); ++i)
    load_to_lds16(base, bs.src[i], __builtin_amdgcn_readfirstlane(l0 + (wave + 4 * i) * 1024));
}

// B operand of tile J for token group u, token 16 u + c.  FP8: bytes K =
// 16 g .. 16 g + 15 (chunk 8 J + g) and K = 64 + 16 g .. (chunk 8 J + 4 + g).
// FP4 (established with one-hot probes, like the A layout): elements K =
// 32 g .. 32 g + 31, low nibble first (chunk 4 J + g); the upper half of the
// operand is unused.
template <int BF>
__device__ __forceinline__ i32x8 read_b(const uint8_t* buf, int u, int J) {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const uint8_t* r = buf + (16 * u + c) * row_bytes<BF>();
  if constexpr (BF == kFmtFp4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(r + 16 * ((4 * J + g) ^ c));
    return i32x8{int(v[0]), int(v[1]), int(v[2]), int(v[3]), 0, 0, 0, 0};
  } else {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(r + 16 * ((8 * J + g) ^ c));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(r + 16 * ((8 * J + 4 + g) ^ c));
    return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                 int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
  }
}

// The contraction of one tile over nkq super-steps, for the first NSub
// 16-token groups.  B (activation codes) is double-buffered in LDS; A
// (weights) is single-buffered in registers and reloaded tile by tile: tile
// J of step kq + 1 is requested as soon as the MFMAs of tile J of step kq
// have read it, so each weight load has a whole step to arrive while only
// one step's weights occupy registers; the exponent dwords of A and B (a
// few registers) are double-buffered and requested at the start of the step
// before the one that uses them.  B operands are read from LDS two (tile, token
// group) pairs ahead of the MFMAs that use them.  Every wave issues the same loads in the same
// order, so one counted wait per step covers the staging.
template <int NSub, int BF, typename Row, typename SRow>
__device__ __forceinline__ void gemm_tile_n(f32x4 (&acc)[kNS][kSub], const AStreams& st, int nkq,
                                            uint8_t* lds, const uint8_t* cbase,
                                            const uint8_t* sbase, Row row, SRow srow) {
#pragma unroll
  for (int s = 0; s < kNS; ++s)
#pragma unroll
    for (int u = 0; u < kSub; ++u) acc[s][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  BStage<NSub, BF> bs;
  prepare_b(bs, cbase, sbase, row, srow);
  ATiles a;
  uint32_t sb[NSub];
  stage_b(lds, 0, bs);
  load_a(a, st, 0);
#pragma unroll
  for (int u = 0; u < NSub; ++u) sb[u] = *reinterpret_cast<const uint32_t*>(bs.sbase + bs.scl[u]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto step = [&](int kq, auto reload) {
    constexpr bool kReload = decltype(reload)::value;
    constexpr int kGroups = 4 * NSub;  // (tile J, token group u) pairs, J major
    const uint8_t* cur = lds + (kq & 1) * stage_bytes<BF>();
    const int kn = kq + 1;
    uint32_t as_n[kNS], sb_n[NSub];  // exponent dwords of step kq + 1
    if constexpr (kReload) {
      stage_b(lds + (kn & 1) * stage_bytes<BF>(), kn, bs);
#pragma unroll
      for (int s = 0; s < kNS; ++s)
        as_n[s] = *reinterpret_cast<const uint32_t*>(st.scl[s] + 4 * kn + st.lane_scl);
#pragma unroll
      for (int u = 0; u < NSub; ++u)
        sb_n[u] = *reinterpret_cast<const uint32_t*>(bs.sbase + 16 * kn + bs.scl[u]);
    }
    i32x8 b[3];  // B operands of groups gi, gi + 1, gi + 2
    b[0] = read_b<BF>(cur, 0, 0);
    if (kGroups > 1) b[1] = read_b<BF>(cur, 1 % NSub, 1 / NSub);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      const int J = gi / NSub, u = gi % NSub;
      if (gi + 2 < kGroups) b[(gi + 2) % 3] = read_b<BF>(cur, (gi + 2) % NSub, (gi + 2) / NSub);
#pragma unroll
      for (int s = 0; s < kNS; ++s) {
        switch (J) {  // opsel J is an immediate
          case 0: acc[s][u] = mma<0, BF>(a.w[s][0], b[gi % 3], acc[s][u], a.s[s], sb[u]); break;
          case 1: acc[s][u] = mma<1, BF>(a.w[s][1], b[gi % 3], acc[s][u], a.s[s], sb[u]); break;
          case 2: acc[s][u] = mma<2, BF>(a.w[s][2], b[gi % 3], acc[s][u], a.s[s], sb[u]); break;
          default: acc[s][u] = mma<3, BF>(a.w[s][3], b[gi % 3], acc[s][u], a.s[s], sb[u]); break;
        }
      }
      if constexpr (kReload) {
        if (u == NSub - 1) {
#pragma unroll
          for (int s = 0; s < kNS; ++s)
            a.w[s][J] = *(reinterpret_cast<const u32x4*>(
                st.codes[s] + size_t(min(4 * kn + J, st.nkb - 1)) * 1024 + st.lane_code));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kReload) {
#pragma unroll
      for (int s = 0; s < kNS; ++s) a.s[s] = as_n[s];
#pragma unroll
      for (int u = 0; u < NSub; ++u) sb[u] = sb_n[u];
      // The staging loads for kq + 1 were issued before this step's 20 + NSub
      // exponent and weight loads; vector loads complete in order, so at most
      // 16 outstanding means every staging load has landed in LDS (for either
      // B format: only the number of staging loads before them differs).  A fenced
      // barrier would wait for all loads: the memory model orders the
      // staging's LDS writes with vmcnt(0).
      __builtin_amdgcn_s_waitcnt(kVmcnt16);
      asm volatile("s_barrier" ::: "memory");
    }
  };
  int kq = 0;
  for (; kq + 1 < nkq; ++kq) step(kq, std::true_type{});
  step(kq, std::false_type{});
}

// Only the 16-token column groups that hold tokens are staged and multiplied
// (ntok = the tile's token count, 1 .. kTok); the other groups keep acc = 0.
// All threads of the workgroup must call it.
// BF: the activations' format (kFmtFp8 or kFmtFp4); row(j) and srow(j) give
// token j's code and exponent rows in bytes.
template <int BF, typename Row, typename SRow>
__device__ __forceinline__ void gemm_tile(f32x4 (&acc)[kNS][kSub], const AStreams& st, int nkq,
                                          uint8_t* lds, int ntok, const uint8_t* cbase,
                                          const uint8_t* sbase, Row row, SRow srow) {
  static_assert(kSub == 4, "one instantiation per group count");
  switch (__builtin_amdgcn_readfirstlane((ntok + 15) / 16)) {
    case 1: gemm_tile_n<1, BF>(acc, st, nkq, lds, cbase, sbase, row, srow); break;
    case 2: gemm_tile_n<2, BF>(acc, st, nkq, lds, cbase, sbase, row, srow); break;
    case 3: gemm_tile_n<3, BF>(acc, st, nkq, lds, cbase, sbase, row, srow); break;
    default: gemm_tile_n<4, BF>(acc, st, nkq, lds, cbase, sbase, row, srow); break;
  }
}

}  // namespace mx
}  // namespace moe
