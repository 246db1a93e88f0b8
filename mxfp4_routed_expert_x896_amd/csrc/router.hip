// Router for decode-sized batches: bf16 logits GEMV, then a wavefront top-k
// with sigmoid scores renormalised over the selected experts.
//
// Deltafin README ("An experiment in running Kimi K3 ..."), "How it works":
// per token and layer the router picks 16 of the 896 routed experts.  The
// scoring rule (sigmoid, ties to the lower index, weights = selected scores
// over their sum) is the reading stated in include/moe_mxfp4.h.
#include "common.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace moe {

namespace {

constexpr int kRouterWaves = 4;   // one expert row per wave
constexpr int kRouterTokens = 4;  // tokens staged in LDS per pass

// logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]).
// Each wave keeps one router row in registers (16-byte chunks c = lane + 64 i)
// and sweeps the tokens, which are staged in LDS kRouterTokens at a time.
template <int NCH>
__global__ __launch_bounds__(kRouterWaves * kWave) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int T, int H, int E) {
  extern __shared__ u32x4 xs[];  // [kRouterTokens][H / 8]
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * kRouterWaves + wave;
  const int nch = H / 8;
  const bool live = e < E;

  u32x4 w[NCH];
  const u32x4* wrow = reinterpret_cast<const u32x4*>(wr + size_t(live ? e : 0) * H);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + kWave * i;
    w[i] = (live && c < nch) ? __builtin_nontemporal_load(wrow + c) : u32x4{0, 0, 0, 0};
  }
  const float b = (live && bias != nullptr) ? bias[e] : 0.0f;

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
      if (live && lane == 0) logits[size_t(t0 + tt) * E + e] = acc + b;
    }
  }
}

// Orderable key: larger logit first, then lower expert index.  Valid keys
// are never 0 (the low word is ~e with e < 1024), so 0 marks "taken".
__device__ __forceinline__ uint64_t topk_key(float l, int e) {
  uint32_t u = __float_as_uint(l);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(u) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(e));
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  uint32_t u = uint32_t(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// Top-k of one token's logits by one wave (all 64 lanes active): k rounds
// of a wave-wide arg-max over the E <= 1024 logits (16 per lane), then
// s = sigmoid(l) and w = s / sum(s).  Selecting on the fp32 logit is the
// same order as on the sigmoid score, without its saturation ties.
__device__ __forceinline__ void select_token(const float* __restrict__ lrow, int E, int k,
                                             int32_t* __restrict__ ids, float* __restrict__ wout) {
  const int lane = threadIdx.x % kWave;
  uint64_t key[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + kWave * i;
    key[i] = e < E ? topk_key(lrow[e], e) : 0ull;
  }
  int my_id = 0;
  float my_logit = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = int(0xFFFFFFFFu - uint32_t(best));
    if (lane == j) {
      my_id = e;
      my_logit = key_logit(best);
    }
    if ((e % kWave) == lane) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i == e / kWave) key[i] = 0ull;
    }
  }
  const float s = lane < k ? 1.0f / (1.0f + expf(-my_logit)) : 0.0f;
  const float tot = wave_sum(s);
  if (lane < k) {
    ids[lane] = my_id;
    wout[lane] = s / tot;
  }
}

// One wave per token, four tokens per workgroup (any T).
__global__ __launch_bounds__(4 * kWave) void router_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ wout) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  select_token(logits + size_t(t) * E, E, k, ids + size_t(t) * k, wout + size_t(t) * k);
}

// Decode batches: one workgroup selects every token's experts (16 waves,
// tokens round-robin) and then builds the token -> expert plan, saving a
// launch between the router and the expert kernels.
__global__ __launch_bounds__(kPlanThreads) void router_select_plan_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ wout, Plan plan, int* zero, int n_zero) {
  for (int t = threadIdx.x / kWave; t < T; t += kPlanThreads / kWave)
    select_token(logits + size_t(t) * E, E, k, ids + size_t(t) * k, wout + size_t(t) * k);
  __syncthreads();
  build_plan(ids, T * k, E, plan, zero, n_zero);
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias,
                                float* logits, int T, int H, int E, hipStream_t stream) {
  const int nch = H / 8;
  const int per_lane = (nch + kWave - 1) / kWave;
  const dim3 grid((E + kRouterWaves - 1) / kRouterWaves);
  const dim3 block(kRouterWaves * kWave);
  const size_t lds = size_t(kRouterTokens) * H * sizeof(uint16_t);
  if (per_lane <= 4)
    hipLaunchKernelGGL(router_logits_kernel<4>, grid, block, lds, stream, x, wr, bias, logits, T, H, E);
  else if (per_lane <= 8)
    hipLaunchKernelGGL(router_logits_kernel<8>, grid, block, lds, stream, x, wr, bias, logits, T, H, E);
  else
    hipLaunchKernelGGL(router_logits_kernel<16>, grid, block, lds, stream, x, wr, bias, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_router_select_plan(const float* logits, int T, int E, int k, int32_t* ids,
                                     float* w, Plan plan, int* zero, int n_zero,
                                     hipStream_t stream) {
  hipLaunchKernelGGL(router_select_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, logits, T,
                     E, k, ids, w, plan, zero, n_zero);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                              hipStream_t stream) {
  hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(4 * kWave), 0, stream, logits, T,
                     E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
