// Prefill path, dense bf16 contractions on the matrix cores
// (v_mfma_f32_16x16x32_bf16): the shared experts' gate/up and down and the
// router logits, for token tiles of 64.
//
// Operand layout (wave64, lane l: g = l / 16, c = l % 16): A lane (c, g)
// holds 8 bf16 of row c, columns 8 g .. 8 g + 7 of a 32-column k-tile --
// lane l of a packed bf16 tile (pack.hip) or 16 bytes of a row-major row;
// B lane (c, g) the same columns of token c; D lane l rows 4 g .. 4 g + 3
// of token c.  A super-step is 4 k-tiles (128 columns).  Tokens are staged
// into LDS with global_load_lds as rows of 256 bytes plus 16 bytes of
// padding (stride 68 dwords, so the 16 lanes of a read phase hit distinct
// banks); columns past the contraction length are zeroed in LDS after the
// loads land, and A tiles past it are clamped to the last valid one, so the
// tail adds nothing.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace bf {

constexpr int kTok = 64;               // tokens per tile
constexpr int kSub = kTok / 16;
constexpr int kStepK = 128;            // contraction columns per super-step
constexpr int kRowB = 2 * kStepK + 16; // staged bytes per token row (+ padding)
constexpr int kChunks = kRowB / 16;    // 17 16-byte chunks per row, the last is padding
constexpr int kStageBytes = kTok * kRowB;  // 17 KiB = 17 wave-wide loads
constexpr int kNS = 4;                 // A streams per wave

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

__device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

struct ATiles {
  u32x4 w[kNS][4];
};

// One wave-wide 16-byte-per-lane load from global memory straight into LDS
// (lane l's bytes land at lds_addr + 16 l), issued as inline assembly so the
// compiler's wait-count bookkeeping, which cannot order such loads against
// ordinary loads and would wait for all of them before the next product,
// does not see it; the caller waits for it explicitly.  s_nop: one wait
// state between writing M0 and a load that reads it.
__device__ __forceinline__ void load_to_lds16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_addr)
               : "memory", "m0");
}

// The tile runs on a group of 4 waves: a 4-wave workgroup, or either half
// of an 8-wave one (which then runs two tiles side by side; both halves go
// through the same barriers).
__device__ __forceinline__ int group_wave() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave % 4);
}

// Stages super-step kq of NB token sources (rows of K bf16) into NB LDS
// buffers of kStageBytes: 17 wave-wide loads each, wave w issuing w, w + 4..
// Chunks past K are loaded from the row's last chunk (valid memory) and
// zeroed later by zero_tail.
template <int NB, typename Row>
__device__ __forceinline__ void stage_b(uint8_t* lds, int kq, int K, Row row) {
  const int wave = group_wave();
  const int lane = threadIdx.x % kWave;
  const int last = K / 8 - 1;  // last 16-byte chunk of a row
  const uint32_t l0 = uint32_t(reinterpret_cast<uintptr_t>((lvoid*)lds));
  for (int n = wave; n < kStageBytes / 1024; n += 4) {
    const int chunk = n * 64 + lane;
    const int j = chunk / kChunks, q = chunk % kChunks;
    const int col_chunk = q < 16 ? min(kq * 16 + q, last) : kq * 16;
#pragma unroll
    for (int s = 0; s < NB; ++s)
      load_to_lds16(row(s, j) + 8 * min(col_chunk, last),
                    __builtin_amdgcn_readfirstlane(l0 + s * kStageBytes + n * 1024));
  }
}

// Zeroes the staged columns >= K of super-step kq (only the last step of a
// K that is not a multiple of 128 has any).
template <int NB>
__device__ __forceinline__ void zero_tail(uint8_t* lds, int kq, int K) {
  const int valid = K - kq * kStepK;  // columns of this step inside K
  if (valid >= kStepK) return;
  const int from = max(valid, 0) / 8;  // first 16-byte chunk to clear
  const int per_row = 16 - from;
  for (int i = threadIdx.x % (kWave * 4); i < NB * kTok * per_row; i += kWave * 4) {
    const int s = i / (kTok * per_row), r = i % (kTok * per_row);
    *reinterpret_cast<u32x4*>(lds + s * kStageBytes + (r / per_row) * kRowB +
                              16 * (from + r % per_row)) = u32x4{0, 0, 0, 0};
  }
}

// A weight tile load; the k-tile index passes through an empty asm
// statement so that two requests of the same (clamped) tile stay two loads:
// the counted wait at the end of a step depends on the number of loads
// issued after the staging.  (kt is the same in every lane: a scalar.)
template <typename AAddr>
__device__ __forceinline__ u32x4 a_load(AAddr a, int s, int kt) {
  asm volatile("" : "+s"(kt));
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a(s, kt)));
}

// A super-step of weights: a(s, kt) is the lane's 16-byte address of
// stream s, k-tile kt (already clamped to the valid tiles by the caller).
template <typename AAddr>
__device__ __forceinline__ void load_a(ATiles& t, AAddr a, int kq) {
#pragma unroll
  for (int s = 0; s < kNS; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t.w[s][j] = a_load(a, s, 4 * kq + j);
}

// s_waitcnt vmcnt(16) with expcnt and lgkmcnt left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kVmcnt16 = (1 << 14) | (7 << 4) | (15 << 8);
static_assert(kNS * 4 >= 16, "a step issues at least 16 ordinary loads after its staging");

// acc[s][u] = sum over the K columns of A stream s x (sum over the NB token
// sources) for token columns 16 u .. 16 u + 15.  lds: NB x 2 stage buffers.
// B (tokens) is double-buffered in LDS; A (weights) is single-buffered in
// registers and reloaded k-tile by k-tile: k-tile j of step kq + 1 is
// requested as soon as the products of k-tile j of step kq have read it, so
// each weight load has a whole step to arrive.  The staging loads of step
// kq + 1 precede the step's 16 weight loads, and vector loads complete in
// order, so one counted wait (at most 16 outstanding) per step covers them.
// All threads of the workgroup must call it.
template <int NB, typename AAddr, typename Row>
__device__ __forceinline__ void gemm_tile(f32x4 (&acc)[kNS][kSub], AAddr a, int K, uint8_t* lds,
                                          Row row) {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
#pragma unroll
  for (int s = 0; s < kNS; ++s)
#pragma unroll
    for (int u = 0; u < kSub; ++u) acc[s][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int nkq = (K + kStepK - 1) / kStepK;
  constexpr int kBuf = NB * kStageBytes;
  const bool tail = K % kStepK != 0;  // the last step has columns past K
  ATiles at;
  stage_b<NB>(lds, 0, K, row);
  load_a(at, a, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tail && nkq == 1) {
    zero_tail<NB>(lds, 0, K);
    __syncthreads();
  }
  // the last step has nothing to reload; a runtime condition around the
  // loads would make the compiler wait for all of them at the next step
  auto step = [&](int kq, auto reload) {
    constexpr bool kReload = decltype(reload)::value;
    const uint8_t* cur = lds + (kq & 1) * kBuf;
    uint8_t* nxt = lds + ((kq + 1) & 1) * kBuf;
    if constexpr (kReload) stage_b<NB>(nxt, kq + 1, K, row);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
#pragma unroll
        for (int s2 = 0; s2 < NB; ++s2) {
          const u32x4 b = *reinterpret_cast<const u32x4*>(cur + s2 * kStageBytes +
                                                          (16 * u + c) * kRowB + 64 * j + 16 * g);
#pragma unroll
          for (int s = 0; s < kNS; ++s) acc[s][u] = mma(at.w[s][j], b, acc[s][u]);
        }
      }
      if constexpr (kReload) {
#pragma unroll
        for (int s = 0; s < kNS; ++s)
          at.w[s][j] = a_load(a, s, 4 * (kq + 1) + j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kReload) {
      // a fenced barrier would wait for every load (the memory model orders
      // the staging's LDS writes with vmcnt(0))
      __builtin_amdgcn_s_waitcnt(kVmcnt16);
      asm volatile("s_barrier" ::: "memory");
      if (tail && kq + 2 == nkq) {
        zero_tail<NB>(nxt, kq + 1, K);
        __syncthreads();
      }
    }
  };
  int kq = 0;
  for (; kq + 1 < nkq; ++kq) step(kq, std::true_type{});
  step(kq, std::false_type{});
}

}  // namespace bf
}  // namespace moe
