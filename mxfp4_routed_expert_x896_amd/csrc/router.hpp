// Router device routines: the bf16 logits GEMV and the per-token top-k with
// sigmoid scores renormalised over the selected experts.
//
// Deltafin README ("An experiment in running Kimi K3 ..."), "How it works":
// per token and layer the router picks 16 of the 896 routed experts.  The
// scoring rule (sigmoid, ties to the lower index, weights = selected scores
// over their sum) is the reading stated in include/moe_mxfp4.h.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kRouterTokens = 2;  // tokens staged in LDS per pass of the logits routine

// logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]) for the four experts
// e = 4 b .. 4 b + 3 of workgroup b (one per wave, 256 threads).  Each wave
// keeps its router row in registers (16-byte chunks c = lane + 64 i) and
// sweeps the tokens, staged in LDS kRouterTokens at a time (xs holds
// kRouterTokens * H bf16).  Every thread of the workgroup must call it.
template <int NCH>
__device__ __forceinline__ void router_logits_rows(const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ wr,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits, int T, int H, int E,
                                                   int b, u32x4* xs) {
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int lane = threadIdx.x % kWave;
  const int e = b * 4 + wave;
  const int nch = H / 8;
  const bool live = e < E;

  u32x4 w[NCH];
  const u32x4* wrow = reinterpret_cast<const u32x4*>(wr + size_t(live ? e : 0) * H);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + kWave * i;
    w[i] = (live && c < nch) ? __builtin_nontemporal_load(wrow + c) : u32x4{0, 0, 0, 0};
  }
  const float bv = (live && bias != nullptr) ? bias[e] : 0.0f;

  for (int t0 = 0; t0 < T; t0 += kRouterTokens) {
    const int nt = min(kRouterTokens, T - t0);
    __syncthreads();
    const u32x4* xsrc = reinterpret_cast<const u32x4*>(x + size_t(t0) * H);
    for (int i = threadIdx.x; i < nt * nch; i += blockDim.x) xs[i] = xsrc[i];
    __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + kWave * i;
        if (c < nch) {
          const u32x4 xv = xs[tt * nch + c];
          acc = dot2_bf16(w[i][0], xv[0], acc);
          acc = dot2_bf16(w[i][1], xv[1], acc);
          acc = dot2_bf16(w[i][2], xv[2], acc);
          acc = dot2_bf16(w[i][3], xv[3], acc);
        }
      }
      acc = wave_sum(acc);
      if (live && lane == 0) logits[size_t(t0 + tt) * E + e] = acc + bv;
    }
  }
}

// Orderable 32-bit image of a float: a > b as floats iff ord(a) > ord(b) as
// unsigned (finite values and infinities); never 0 for a finite value.
__device__ __forceinline__ uint32_t ord_f32(float l) {
  const uint32_t u = __float_as_uint(l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord_f32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32_step(uint32_t v) {
  const uint32_t o = dpp_or_zero<CTRL, ROW_MASK>(v);
  return o > v ? o : v;
}

// Maximum of an unsigned 32-bit value over all 64 lanes; result in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32_step<0xB1, 0xF>(v);
  v = dpp_max_u32_step<0x4E, 0xF>(v);
  v = dpp_max_u32_step<0x141, 0xF>(v);
  v = dpp_max_u32_step<0x140, 0xF>(v);
  v = dpp_max_u32_step<0x142, 0xA>(v);
  v = dpp_max_u32_step<0x143, 0xC>(v);
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

// Top-k (k <= 32) of one token's E <= 1024 logits by one wave (all 64 lanes
// active): lane j < k receives the j-th selected expert (score descending,
// ties to the lower expert index) in id and w = sigmoid(l) / sum over the
// selected.  Selecting on the fp32 logit is the same order as on the
// sigmoid score, without its saturation ties.
//
// Fast path: every lane keeps its 4 best (value, index) candidates sorted;
// each round takes the wave-wide best head (32-bit DPP max, ties resolved
// by the lowest index) and pops it from its lane.  If some lane runs out of
// candidates before the last round, its fifth key might belong to the top-k:
// the token is then redone exactly by k rounds over all 16 keys per lane.
__device__ __forceinline__ void select_token(const float* __restrict__ lrow, int E, int k,
                                             int& id, float& w) {
  const int lane = threadIdx.x % kWave;
  uint32_t val[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + kWave * i;
    val[i] = e < E ? ord_f32(lrow[e]) : 0u;
  }
  // per-lane sorted top 4; indices rise with i, so strict > keeps ties in
  // index order
  uint32_t cv[4] = {0u, 0u, 0u, 0u};
  int ci[4] = {1 << 20, 1 << 20, 1 << 20, 1 << 20};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t v = val[i];
    const int e = lane + kWave * i;
    const bool b0 = v > cv[0], b1 = v > cv[1], b2 = v > cv[2], b3 = v > cv[3];
    cv[3] = b2 ? cv[2] : (b3 ? v : cv[3]);
    ci[3] = b2 ? ci[2] : (b3 ? e : ci[3]);
    cv[2] = b1 ? cv[1] : (b2 ? v : cv[2]);
    ci[2] = b1 ? ci[1] : (b2 ? e : ci[2]);
    cv[1] = b0 ? cv[0] : (b1 ? v : cv[1]);
    ci[1] = b0 ? ci[0] : (b1 ? e : ci[1]);
    cv[0] = b0 ? v : cv[0];
    ci[0] = b0 ? e : ci[0];
  }
  int my_id = 0;
  uint32_t my_val = 0;
  int used = 0;
  bool overflow = false;
  for (int j = 0; j < k; ++j) {
    const uint32_t m = wave_max_u32(cv[0]);
    const uint64_t tied = __ballot(cv[0] == m);
    int win_lane, win_id;
    if (__popcll(tied) == 1) {
      win_lane = __ffsll((unsigned long long)tied) - 1;
      win_id = __builtin_amdgcn_readlane(ci[0], win_lane);
    } else {  // equal logits in several lanes: the lowest expert index wins
      const uint32_t inv = cv[0] == m ? ~uint32_t(ci[0]) : 0u;
      win_id = int(~wave_max_u32(inv));
      win_lane = win_id % kWave;
    }
    if (lane == j) {
      my_id = win_id;
      my_val = m;
    }
    if (lane == win_lane) {
      cv[0] = cv[1], ci[0] = ci[1];
      cv[1] = cv[2], ci[1] = ci[2];
      cv[2] = cv[3], ci[2] = ci[3];
      cv[3] = 0u, ci[3] = 1 << 20;
      ++used;
      if (used == 4 && j < k - 1) overflow = true;
    }
  }
  if (__ballot(overflow) != 0) {
    // exact slow path: k rounds over all keys, 64-bit (value, ~index) keys
    uint64_t key[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + kWave * i;
      key[i] = val[i] == 0u ? 0ull
                            : ((uint64_t(val[i]) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(e)));
    }
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e = int(0xFFFFFFFFu - uint32_t(best));
      if (lane == j) {
        my_id = e;
        my_val = uint32_t(best >> 32);
      }
      if ((e % kWave) == lane) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i == e / kWave) key[i] = 0ull;
      }
    }
  }
  const float s = lane < k ? 1.0f / (1.0f + expf(-unord_f32(my_val))) : 0.0f;
  const float tot = wave_sum(s);
  id = my_id;
  w = s / tot;
}

}  // namespace moe
