// Token -> expert grouping, as a device routine for one 1024-thread
// workgroup (used by the stand-alone plan kernel and by the fused
// select-and-plan kernel of the router).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kPlanThreads = 1024;

// Inclusive scan of one int per thread across the 1024-thread workgroup.
__device__ __forceinline__ int block_inclusive_scan(int v, int* warp_tot) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) warp_tot[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int s = lane < kPlanThreads / kWave ? warp_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(s, off, kWave);
      if (lane >= off) s += o;
    }
    if (lane < kPlanThreads / kWave) warp_tot[lane] = s;
  }
  __syncthreads();
  const int add = wave > 0 ? warp_tot[wave - 1] : 0;
  __syncthreads();
  return v + add;
}

// Builds `plan` from ids[n_pairs] (E <= 1024) and zeroes zero[0..n_zero).
// Ids outside [0, E) are clamped so no access leaves the buffers; such
// routings are the caller's error.  Pairs of one expert are listed in the
// order the workgroup's atomics hand out slots (the results do not depend
// on it: every pair is computed the same way wherever it sits).
__device__ __forceinline__ void build_plan(const int32_t* ids, int n_pairs, int E, Plan plan,
                                           int* zero, int n_zero) {
  __shared__ int cnt[1024];
  __shared__ int fill[1024];
  __shared__ int warp_tot[kPlanThreads / kWave];
  const int tid = threadIdx.x;
  for (int i = tid; i < n_zero; i += kPlanThreads) zero[i] = 0;
  cnt[tid] = 0;
  __syncthreads();
  for (int p = tid; p < n_pairs; p += kPlanThreads) {
    const int e = min(max(ids[p], 0), E - 1);
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  const int incl = block_inclusive_scan(c, warp_tot);
  const int flag = c > 0 ? 1 : 0;
  const int aincl = block_inclusive_scan(flag, warp_tot);
  const int excl = incl - c;
  if (flag) {
    plan.active[aincl - 1] = tid;
    plan.act_off[aincl - 1] = excl;
  }
  fill[tid] = excl;
  if (tid == kPlanThreads - 1) {
    plan.n_active[0] = aincl;
    plan.act_off[aincl] = n_pairs;
  }
  __syncthreads();
  for (int p = tid; p < n_pairs; p += kPlanThreads) {
    const int e = min(max(ids[p], 0), E - 1);
    const int slot = atomicAdd(&fill[e], 1);
    plan.pairs[slot] = p;
  }
}

}  // namespace moe
