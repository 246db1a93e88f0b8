// Token -> expert grouping ("plan") built by one 256-thread workgroup, so
// that each routed expert's weights are streamed once per call however many
// tokens chose it (Deltafin README, "How it works": each token reads only
// the experts it selected; a batch reads the union of their selections).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kPlanThreads = 256;
constexpr int kPlanExperts = 1024;  // largest expert count the plan handles

// Inclusive scan of one int per thread across a 256-thread workgroup.
// wtot: kPlanThreads / kWave ints of LDS; every thread must call it.
__device__ __forceinline__ int block_inclusive_scan(int v, int* wtot) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) wtot[wave] = v;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int w = 0; w < kPlanThreads / kWave; ++w)
    if (w < wave) add += wtot[w];
  __syncthreads();
  return v + add;
}

// Eight routing ids per thread in flight at once (they may come from far
// memory: one round trip per batch instead of per pair): e[j] = the expert
// of pair p0 + j * kPlanThreads + tid, clamped to [0, E), or -1 past
// n_pairs.  The loads are unconditional (clamped index) and taken together;
// a load under a condition would be waited for on its own.
constexpr int kBatch = 8;
template <typename Ids>
__device__ __forceinline__ void batch_ids(Ids ids, int p0, int n_pairs, int E, int (&e)[kBatch]) {
  int v[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    v[j] = ids(min(p0 + j * kPlanThreads + int(threadIdx.x), n_pairs - 1));
#pragma unroll
  for (int j = 0; j < kBatch; ++j) asm volatile("" : "+v"(v[j]));
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    e[j] = p0 + j * kPlanThreads + int(threadIdx.x) < n_pairs ? min(max(v[j], 0), E - 1) : -1;
}

// Builds `plan` from the routing ids(p), p < n_pairs (E <= kPlanExperts),
// including the list of token tiles (kPlanTileTokens pairs of one expert,
// in slot order), and zeroes zero[0 .. n_zero).  ids(p) is a callback so the routing can be
// read either plainly or through the device-coherent level.  Ids outside
// [0, E) are clamped, so nothing is read or written out of bounds; such a
// routing is the caller's error.  The pairs of one expert are listed in the
// order the LDS atomics hand out slots; no result depends on that order
// (each pair is computed on its own and combined by slot index).
template <typename Ids>
__device__ void build_plan(Ids ids, int n_pairs, int E, Plan plan, int* zero, int n_zero) {
  __shared__ int cnt[kPlanExperts];
  __shared__ int wtot[kPlanThreads / kWave];
  const int tid = threadIdx.x;
  for (int i = tid; i < n_zero; i += kPlanThreads) zero[i] = 0;
  for (int i = tid; i < kPlanExperts; i += kPlanThreads) cnt[i] = 0;
  __syncthreads();
  for (int p0 = 0; p0 < n_pairs; p0 += kBatch * kPlanThreads) {
    int e[kBatch];
    batch_ids(ids, p0, n_pairs, E, e);
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (e[j] >= 0) atomicAdd(&cnt[e[j]], 1);
  }
  __syncthreads();
  // Thread tid owns experts 4 tid .. 4 tid + 3.
  int c[4], s = 0, a = 0, m = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = cnt[4 * tid + q];
    s += c[q];
    a += c[q] > 0 ? 1 : 0;
    m += (c[q] + kPlanTileTokens - 1) / kPlanTileTokens;
  }
  const int s_incl = block_inclusive_scan(s, wtot);
  const int a_incl = block_inclusive_scan(a, wtot);
  const int m_incl = block_inclusive_scan(m, wtot);
  int off = s_incl - s, ao = a_incl - a, mo = m_incl - m;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    if (c[q] > 0) {
      for (int j = 0; j * kPlanTileTokens < c[q]; ++j) plan.mtiles[mo++] = (ao << 16) | j;
      plan.active[ao] = e;
      plan.act_off[ao] = off;
      ++ao;
    }
    cnt[e] = off;  // from here on: next free slot of expert e
    off += c[q];
  }
  if (tid == kPlanThreads - 1) {
    plan.n_active[0] = a_incl;
    plan.act_off[a_incl] = n_pairs;
    plan.n_mtiles[0] = m_incl;
  }
  __syncthreads();
  for (int p0 = 0; p0 < n_pairs; p0 += kBatch * kPlanThreads) {
    int e[kBatch];
    batch_ids(ids, p0, n_pairs, E, e);
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (e[j] >= 0) plan.pairs[atomicAdd(&cnt[e[j]], 1)] = p0 + j * kPlanThreads + tid;
  }
}

}  // namespace moe
