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
      // through the coherent level: a top-k workgroup of the same launch may
      // read them (see select_waits in layer.hip)
      if (live && lane == 0) store_coherent(&logits[size_t(t0 + tt) * E + e], acc + bv);
    }
  }
}

// Orderable 32-bit image of a float: a > b as floats iff ord(a) > ord(b) as
// unsigned (finite values and infinities); never 0 for a finite value.
__device__ __forceinline__ uint32_t ord_f32(float l) {
  const uint32_t u = __float_as_uint(l + 0.0f);  // -0 + 0 = +0: the zeros tie
  // negative: all bits flipped; positive: sign bit set
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
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

// Candidate keys a wave keeps in LDS during one token's top-k.
constexpr int kSelCap = 256;

// Per-wave LDS of select_token.
struct alignas(16) SelectScratch {
  uint32_t lmax[kWave];      // each lane's largest key
  uint64_t cand[kSelCap + kWave];  // candidate (value, index) keys; the last kWave
                                   // entries take the other lanes' stores
  uint64_t top[32];          // the selected keys by rank
};

// Orders this wave's LDS stores before its later LDS loads (a wave's LDS
// accesses are carried out in program order; this keeps the compiler from
// moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exclusive prefix sum over the lanes of a count 0 <= v < 32, and the
// total, from one ballot per bit.
__device__ __forceinline__ int wave_prefix_small(int v, int& total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit) {
    const uint64_t m = __ballot((v >> bit) & 1);
    const int below = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
    pre += below << bit;
    tot += __popcll(m) << bit;
  }
  total = tot;
  return pre;
}

// Top-k (k <= 32) of one token's E <= 1024 logits by one wave (all 64 lanes
// active): lane j < k receives the j-th selected expert (score descending,
// ties to the lower expert index) in id and w = sigmoid(l) / sum over the
// selected.  Selecting on the fp32 logit is the same order as on the
// sigmoid score, without its saturation ties.
//
// Each key is the pair (ordered logit, inverted index), unique per expert,
// so "larger key" is exactly the selection order.  Lane l holds experts
// l + 64 i.  The k-th largest of the 64 per-lane maxima is a lower bound M
// on the k-th largest logit (k lanes hold a value >= M), so every selected
// expert has a logit >= M.  The experts at or above M (a few more than k
// for any spread-out logits) are gathered in LDS and each one's rank among
// them -- which equals its rank among all experts, since any larger key is
// also at or above M -- is counted directly; ranks below k are the
// selection.  If more than kSelCap experts reach M (heavy ties), the token
// is redone exactly by k rounds of a wave-wide maximum over all keys.
// kCoherent: the logits were written in the same launch (read past L2).
// kSplit > 1: lrow is the first of kSplit partial rows pstride floats apart,
// summed in order.
// kSelBias: the bias takes part in the choice only (DeepSeek-V3 report,
// section 2.1.2): the key is sigmoid(l) + sbias[e] instead of l, and the
// weights still come from the unbiased sigmoid(l), recomputed for the
// chosen experts from the same logits.  scale multiplies every weight.
template <bool kCoherent = false, int kSplit = 1, bool kSelBias = false>
__device__ __forceinline__ void select_token(const float* __restrict__ lrow, size_t pstride,
                                             int E, int k, int& id, float& w,
                                             SelectScratch& sc,
                                             const float* __restrict__ sbias = nullptr,
                                             float scale = 1.0f) {
  const int lane = threadIdx.x % kWave;
  uint32_t val[16];
  // unconditional loads (clamped address), so all of them are in flight at
  // once; a load under a condition would be waited for on its own
  float lv[kSplit][16];
#pragma unroll
  for (int q = 0; q < kSplit; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float* p = lrow + q * pstride + min(lane + kWave * i, E - 1);
      lv[q][i] = kCoherent ? load_coherent(p) : *p;
    }
  // the values are taken here, so no load is moved under the condition below
#pragma unroll
  for (int q = 0; q < kSplit; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(lv[q][i]));
#pragma unroll
  for (int q = 1; q < kSplit; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) lv[0][i] += lv[q][i];
  if constexpr (kSelBias) {
    float bv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) bv[i] = sbias[min(lane + kWave * i, E - 1)];
#pragma unroll
    for (int i = 0; i < 16; ++i) lv[0][i] = 1.0f / (1.0f + expf(-lv[0][i])) + bv[i];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) val[i] = lane + kWave * i < E ? ord_f32(lv[0][i]) : 0u;
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = val[i] > mx ? val[i] : mx;
  sc.lmax[lane] = mx;
  wave_lds_sync();
  // number of lanes whose maximum is >= this lane's; the threshold is the
  // largest maximum that at least k lanes reach
  int ge = 0;
#pragma unroll
  for (int j = 0; j < kWave; j += 4) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(&sc.lmax[j]);
#pragma unroll
    for (int t = 0; t < 4; ++t) ge += q[t] >= mx ? 1 : 0;
  }
  const uint32_t M = wave_max_u32(ge >= k ? mx : 0u);
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) cnt += (lane + kWave * i < E && val[i] >= M) ? 1 : 0;
  int total;
  int off = wave_prefix_small(cnt, total);
  int my_id = 0;
  uint32_t my_val = 0;
  const bool overflow = total > kSelCap;
  if (!overflow) {
    // every lane stores each of its keys: candidates to the next free slot,
    // the others to the lane's own slot past the candidates (no branches)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + kWave * i;
      const bool is_c = e < E && val[i] >= M;
      sc.cand[is_c ? off : kSelCap + lane] =
          (uint64_t(val[i]) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(e));
      off += is_c ? 1 : 0;
    }
    wave_lds_sync();
    for (int c = lane; c < total; c += kWave) {
      const uint64_t key = sc.cand[c];
      int r = 0;
      // eight keys per pass, loaded together (reads past total stay inside
      // the array and are not counted)
      for (int t0 = 0; t0 < total; t0 += 8) {
        uint64_t q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = sc.cand[t0 + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) r += (t0 + u < total && q[u] > key) ? 1 : 0;
      }
      if (r < k) sc.top[r] = key;
    }
    wave_lds_sync();
    if (lane < k) {
      const uint64_t key = sc.top[lane];
      my_val = uint32_t(key >> 32);
      my_id = int(0xFFFFFFFFu - uint32_t(key));
    }
  }
  if (overflow) {
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
  float l = unord_f32(my_val);
  if constexpr (kSelBias) {
    // the chosen expert's logit, summed in the same order as above
    l = 0.0f;
#pragma unroll
    for (int q = 0; q < kSplit; ++q) {
      const float* p = lrow + q * pstride + my_id;
      l += kCoherent ? load_coherent(p) : *p;
    }
  }
  const float s = lane < k ? 1.0f / (1.0f + expf(-l)) : 0.0f;
  const float tot = wave_sum(s);
  id = my_id;
  w = s / tot * scale;
}

}  // namespace moe
