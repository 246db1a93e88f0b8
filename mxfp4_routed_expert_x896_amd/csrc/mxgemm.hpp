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
// exponents in one dword, so tile j of the super-step uses opsel j.  The staged
// activations keep the same convention: per token and super-step, 16 scale
// bytes ordered [g][j] (block 16 kq + 4 j + g at byte 4 g + j), so lane g's
// dword holds its four tiles' exponents.
//
// Work split: a workgroup of 8 waves takes one token tile (up to kTok = 96
// tokens of one expert) and 8 x 4 row groups of 16 weight rows; each wave
// keeps 4 row groups x 6 token groups of fp32 accumulators (96 registers)
// and streams its own weight tiles into registers, while the tile's
// activation codes and exponents are staged in LDS for all waves.  Per
// 16x16x128 MFMA that is 235 bytes brought into the CU (a 64-token, 4-wave
// tile needed 384).  The contraction advances in steps of two MFMA tiles
// (256 columns): weight tiles are double-buffered in registers and
// requested two steps ahead, activations are triple-buffered in LDS and
// staged two steps ahead, so every load has about two steps (96 MFMAs per
// SIMD for a full tile) to arrive.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace mx {

constexpr int kTok = kPlanTileTokens;  // tokens (B columns) per tile
constexpr int kSub = kTok / 16;        // 16-token MFMA column groups per tile
constexpr int kWaves = kMxThreads / kWave;
constexpr int kStepK = 256;            // contraction columns per step (2 MFMA tiles)
constexpr int kNS = 4;                 // A streams (16-row groups x matrices) per wave
constexpr int kExpBytes = kTok * 16;   // a stage's activation exponents: 16 bytes per token
constexpr int kStages = 3;             // LDS stage buffers

// B (activation) formats: the MFMA's blgp operand code.
constexpr int kFmtFp8 = 0;  // MXFP8: E4M3 codes, one byte per element
constexpr int kFmtFp4 = 4;  // MXFP4: E2M1 codes, two per byte, even element in the low nibble
// Bytes of one token's codes in one step; a stage holds the codes of kTok
// tokens, then their exponents (of the step's 512-column super-step).
template <int BF>
constexpr int row_bytes() { return BF == kFmtFp4 ? kStepK / 2 : kStepK; }
template <int BF>
constexpr int code_bytes() { return kTok * row_bytes<BF>(); }
template <int BF>
constexpr int stage_bytes() { return code_bytes<BF>() + kExpBytes; }
// Code loads (1 KiB each) of one stage for NSub token groups; every wave
// issues the same number of them (the last one repeated where they do not
// divide evenly), so that one counted wait fits all waves.
template <int BF>
constexpr int tokens_per_load() { return 1024 / row_bytes<BF>(); }
template <int NSub, int BF>
constexpr int code_loads() { return 16 * NSub / tokens_per_load<BF>(); }
template <int NSub, int BF>
constexpr int wave_loads() { return (code_loads<NSub, BF>() + kWaves - 1) / kWaves; }
constexpr int kMaxWaveLoads = (16 * kSub / 4 + kWaves - 1) / kWaves;  // FP8, all groups
// LDS of a prefill GEMM workgroup: the stages, then the per-lane staging
// source offsets (kMaxWaveLoads + 1 dwords per thread).
template <int BF>
constexpr int lds_bytes() {
  return kStages * stage_bytes<BF>() + (kMaxWaveLoads + 1) * kMxThreads * 4;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lvoid;

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

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

// Global-memory views of the weight streams.
typedef __attribute__((address_space(1))) const uint8_t gbyte;
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const uint32_t gu32;

// p, known to be the same in every lane, as a scalar global pointer: loads
// then take their base from SGPRs and only the lane's 32-bit offset from a
// VGPR.
__device__ __forceinline__ const gbyte* uniform_gptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const gbyte*>((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const uint8_t*>((uint64_t(hi) << 32) | lo);
}

// Streams of a wave: code tiles of a 16-row group and its exponent dwords
// (per super-step 64 lane dwords, 256 bytes).  The stream bases are uniform
// across the wave; the lane's part is a 32-bit offset shared by all streams
// (16 lane into a code tile, 4 lane into a super-step's exponents).
struct AStreams {
  const gbyte* codes[kNS];
  const gbyte* scl[kNS];
  uint32_t lane_code, lane_scl;
  int nkb;   // code tiles per row group
  int nsup;  // super-steps (exponent dwords per lane)
};

// Code tile kb of stream s (clamped to the last).  The offset passes through
// an empty asm statement so that two requests of the same (clamped) tile in
// one step stay two loads: the waits count them.
__device__ __forceinline__ u32x4 a_tile(const AStreams& st, int s, int kb) {
  uint32_t off = uint32_t(min(kb, st.nkb - 1)) * 1024u + st.lane_code;
  asm volatile("" : "+v"(off));
  // one 32-bit offset (uniform part + lane part) on the scalar base
  return *reinterpret_cast<gu32x4*>(st.codes[s] + off);
}
// Exponent dword of super-step q (tiles 4 q .. 4 q + 3) of stream s.
__device__ __forceinline__ uint32_t a_exps(const AStreams& st, int s, int q) {
  uint32_t off = 256 * uint32_t(min(q, st.nsup - 1)) + st.lane_scl;
  asm volatile("" : "+v"(off));
  return *reinterpret_cast<gu32*>(st.scl[s] + off);
}

// One wave-wide load from global memory (base + lane's off) straight into
// LDS: 16 bytes per lane (lane l's at lds_addr + 16 l), or 4 (at lds_addr +
// 4 l).  Issued as inline assembly so that the compiler's wait-count
// bookkeeping, which cannot order such loads against ordinary loads and
// would then wait for every load before the next MFMA, does not see it: the
// caller waits for it explicitly.  s_nop: one wait state between writing M0
// and a load that reads it.
__device__ __forceinline__ void load_to_lds16(const uint8_t* base, uint32_t off,
                                              uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void load_to_lds4(const uint8_t* base, uint32_t off,
                                             uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// Staged activations, one step per stage.
//   codes: token j's bytes of the step (row_bytes: 256 for FP8, 128 for
//     FP4) as 16-byte chunks, chunk q at slot q ^ (j % 16) (FP8) or
//     q ^ (j % 8) (FP4) of the token's LDS row, so the lanes that read the
//     same chunk of consecutive tokens spread over the banks; one wave-wide
//     load fills 1 KiB (4 FP8 token rows, 8 FP4 ones);
//   exponents: token j's 16 bytes of the step's super-step at code_bytes +
//     16 j, one 4-byte-per-lane load per 16 tokens.
// The global source of each of a wave's loads at step 0, as a 32-bit byte
// offset per lane from the wave-uniform base, is kept in LDS (written once
// per tile, read back at each staging) rather than in registers, which the
// accumulators and weight tiles fill.
template <int BF>
constexpr int slot_mask() { return BF == kFmtFp4 ? 7 : 15; }

template <int NSub, int BF, typename Row, typename SRow>
__device__ __forceinline__ void prepare_b(uint32_t* offs, Row row, SRow srow) {
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int lane = threadIdx.x % kWave;
  constexpr int kChunks = row_bytes<BF>() / 16;  // chunks per token row: 16 (FP8), 8 (FP4)
#pragma unroll
  for (int m = 0; m < wave_loads<NSub, BF>(); ++m) {
    const int i = min(wave + kWaves * m, code_loads<NSub, BF>() - 1);
    const int j = tokens_per_load<BF>() * i + lane / kChunks;
    offs[m * kMxThreads + threadIdx.x] =
        row(j) + 16 * ((lane % kChunks) ^ (j & slot_mask<BF>()));
  }
  const int j = 16 * min(wave, NSub - 1) + lane / 4;
  offs[kMaxWaveLoads * kMxThreads + threadIdx.x] = srow(j) + 4 * (lane % 4);
}

// Stages step kq of the first 16 NSub tokens into buf: every wave issues
// wave_loads + 1 loads.
template <int NSub, int BF>
__device__ __forceinline__ void stage_b(uint8_t* buf, int kq, const uint8_t* cbase,
                                        const uint8_t* sbase, const uint32_t* offs) {
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const uint8_t* base = uniform_ptr(cbase + size_t(kq) * row_bytes<BF>());
  const uint32_t l0 = uint32_t(reinterpret_cast<uintptr_t>((lvoid*)buf));
#pragma unroll
  for (int m = 0; m < wave_loads<NSub, BF>(); ++m) {
    const int i = min(wave + kWaves * m, code_loads<NSub, BF>() - 1);
    load_to_lds16(base, offs[m * kMxThreads + threadIdx.x],
                  __builtin_amdgcn_readfirstlane(l0 + i * 1024));
  }
  load_to_lds4(uniform_ptr(sbase + size_t(kq / 2) * 16), offs[kMaxWaveLoads * kMxThreads + threadIdx.x],
               __builtin_amdgcn_readfirstlane(l0 + code_bytes<BF>() + 256 * min(wave, NSub - 1)));
}

// B operand of step tile J (0, 1) for token group u, token 16 u + c.  FP8:
// bytes K = 16 g .. 16 g + 15 (chunk 8 J + g) and K = 64 + 16 g .. (chunk
// 8 J + 4 + g).  FP4 (established with one-hot probes, like the A layout):
// elements K = 32 g .. 32 g + 31, low nibble first (chunk 4 J + g); the
// upper half of the operand is unused.
//
// The lane's swizzled slot differs from that of chunk g only in the bits
// the tile index and the half set (FP8: bit 2 = upper half, bit 3 = J; FP4:
// bit 2 = J), so a lane keeps one byte offset, its chunk-g slot in its token
// row, and XORs those bits (times 16) into it; the token group is a constant
// folded into each LDS read's immediate offset.
template <int BF>
__device__ __forceinline__ uint32_t b_lane() {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  return c * row_bytes<BF>() + 16 * ((g ^ c) & slot_mask<BF>());
}
template <int BF>
__device__ __forceinline__ i32x8 read_b(const uint8_t* buf, uint32_t bl, int u, int J) {
  if constexpr (BF == kFmtFp4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(buf + (bl ^ (64 * J)) +
                                                    16 * row_bytes<BF>() * u);
    return i32x8{int(v[0]), int(v[1]), int(v[2]), int(v[3]), 0, 0, 0, 0};
  } else {
    const int k = 16 * row_bytes<BF>() * u;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(buf + (bl ^ (128 * J)) + k);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(buf + (bl ^ (128 * J + 64)) + k);
    return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                 int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
  }
}
// B exponent dword of token group u: token 16 u + c, its super-step's 4
// tiles' exponents of lane group g.
template <int BF>
__device__ __forceinline__ uint32_t read_sb(const uint8_t* buf, int u) {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  return *reinterpret_cast<const uint32_t*>(buf + code_bytes<BF>() + 16 * c + 4 * g + 256 * u);
}

// The contraction of one tile over nks steps (nks even: whole super-steps),
// for the first NSub 16-token groups; see the header comment for the
// pipeline.  Step kq uses weight buffer kq % 2 and stage kq % 3, and
// requests the weights of step kq + 2 into its own weight buffer tile by
// tile as the MFMAs release them, and the stage of step kq + 2.  The
// exponent dwords of the weights cover a super-step (two steps) and are
// requested one super-step ahead.
//
// Waits: the staging loads (inline assembly) are not counted by the
// compiler, so every wave issues the same number of them (D) and waits for
// them itself: at the end of step kq the stage of step kq + 1, issued at
// the start of step kq - 1, is followed by 8 + 4 + 8 weight loads and the D
// staging loads of step kq + 2, so vmcnt(20 + D) means it has landed; a
// barrier then covers every wave's.  The compiler's own waits for weight
// loads undercount by the staging in between, which makes them also wait
// for staging issued a step earlier, never for the stage just requested.
template <int NSub, int BF, typename Row, typename SRow>
__device__ __forceinline__ void gemm_tile_n(f32x4 (&acc)[kNS][kSub], const AStreams& st, int nks,
                                            uint8_t* lds, const uint8_t* cbase,
                                            const uint8_t* sbase, Row row, SRow srow) {
  constexpr int D = wave_loads<NSub, BF>() + 1;
  static_assert(20 + D <= 63, "vmcnt range");
#pragma unroll
  for (int s = 0; s < kNS; ++s)
#pragma unroll
    for (int u = 0; u < kSub; ++u) acc[s][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t* offs = reinterpret_cast<uint32_t*>(lds + kStages * stage_bytes<BF>());
  prepare_b<NSub, BF>(offs, row, srow);
  const uint32_t bl = b_lane<BF>();
  u32x4 a[2][kNS][2];  // weight tiles: [step parity][stream][tile of the step]
  uint32_t as[kNS], as_n[kNS];  // exponent dwords of this and the next super-step
  // prologue: stages 0 and 1, weights of steps 0 and 1, exponents of
  // super-step 0 (each lane reads back only the offsets it wrote)
  stage_b<NSub, BF>(lds, 0, cbase, sbase, offs);
  stage_b<NSub, BF>(lds + stage_bytes<BF>(), 1, cbase, sbase, offs);
#pragma unroll
  for (int s = 0; s < kNS; ++s) {
    as[s] = a_exps(st, s, 0);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j) a[p][s][j] = a_tile(st, s, 2 * p + j);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int cs = 0;  // stage of step kq
  // P: kq % 2 (also the half of the super-step: opsel 2 P + J)
  auto step = [&](int kq, auto parity) {
    constexpr int P = decltype(parity)::value;
    constexpr int kGroups = 2 * NSub;  // (tile J, token group u) pairs, J major
    const uint8_t* cur = lds + cs * stage_bytes<BF>();
    const int ns = cs == 0 ? 2 : cs - 1;  // stage of step kq + 2
    stage_b<NSub, BF>(lds + ns * stage_bytes<BF>(), min(kq + 2, nks - 1), cbase, sbase, offs);
    if constexpr (P == 0) {
#pragma unroll
      for (int s = 0; s < kNS; ++s) as_n[s] = a_exps(st, s, kq / 2 + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      const int J = gi / NSub, u = gi % NSub;
      const i32x8 bv = read_b<BF>(cur, bl, u, J);
      const uint32_t sv = read_sb<BF>(cur, u);
#pragma unroll
      for (int s = 0; s < kNS; ++s) {
        if (J == 0)
          acc[s][u] = mma<2 * P, BF>(a[P][s][0], bv, acc[s][u], as[s], sv);
        else
          acc[s][u] = mma<2 * P + 1, BF>(a[P][s][1], bv, acc[s][u], as[s], sv);
      }
      if (u == NSub - 1) {
#pragma unroll
        for (int s = 0; s < kNS; ++s) a[P][s][J] = a_tile(st, s, 2 * (kq + 2) + J);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (P == 1) {
#pragma unroll
      for (int s = 0; s < kNS; ++s) as[s] = as_n[s];
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(20 + D));
    asm volatile("s_barrier" ::: "memory");
    cs = cs == 2 ? 0 : cs + 1;
  };
  for (int kq = 0; kq < nks; kq += 2) {
    step(kq, std::integral_constant<int, 0>{});
    step(kq + 1, std::integral_constant<int, 1>{});
  }
  // the loads past the last step (clamped, unused) are left to land before
  // the caller's epilogue reuses nothing of them: drain them here
  __builtin_amdgcn_s_waitcnt(0);
}

// Only the 16-token column groups that hold tokens are staged and multiplied
// (ntok = the tile's token count, 1 .. kTok); the other groups keep acc = 0.
// All threads of the workgroup must call it.  nks: steps (even).
// BF: the activations' format (kFmtFp8 or kFmtFp4); row(j) and srow(j) give
// token j's code and exponent rows in bytes (0 <= j < kTok), the code row
// counted in steps (row(j) + kq row_bytes is step kq of token j).
template <int BF, typename Row, typename SRow>
__device__ __forceinline__ void gemm_tile(f32x4 (&acc)[kNS][kSub], const AStreams& st, int nks,
                                          uint8_t* lds, int ntok, const uint8_t* cbase,
                                          const uint8_t* sbase, Row row, SRow srow) {
  static_assert(kSub == 6, "one instantiation per group count");
  switch (__builtin_amdgcn_readfirstlane((ntok + 15) / 16)) {
    case 1: gemm_tile_n<1, BF>(acc, st, nks, lds, cbase, sbase, row, srow); break;
    case 2: gemm_tile_n<2, BF>(acc, st, nks, lds, cbase, sbase, row, srow); break;
    case 3: gemm_tile_n<3, BF>(acc, st, nks, lds, cbase, sbase, row, srow); break;
    case 4: gemm_tile_n<4, BF>(acc, st, nks, lds, cbase, sbase, row, srow); break;
    case 5: gemm_tile_n<5, BF>(acc, st, nks, lds, cbase, sbase, row, srow); break;
    default: gemm_tile_n<6, BF>(acc, st, nks, lds, cbase, sbase, row, srow); break;
  }
}

}  // namespace mx
}  // namespace moe
