// Token -> expert grouping for batched decode: per-expert counts, the list of
// experts that received tokens, and the pair ids grouped by expert, so that
// every expert's weights stream from HBM once per call however many tokens
// chose it.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kPlanThreads = 1024;

// Inclusive scan of one int per thread across the 1024-thread block.
__device__ int block_inclusive_scan(int v, int* warp_tot) {
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

// Single workgroup.  Ids outside [0, E) are clamped so no access leaves the
// buffers; such routings are the caller's error.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ ids,
                                                            int n_pairs, int E, Plan plan) {
  __shared__ int cnt[1024];
  __shared__ int fill[1024];
  __shared__ int warp_tot[kPlanThreads / kWave];
  const int tid = threadIdx.x;
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

}  // namespace

hipError_t launch_plan(const int32_t* ids, int n_pairs, int E, Plan plan, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, ids, n_pairs, E, plan);
  return hipGetLastError();
}

}  // namespace moe
