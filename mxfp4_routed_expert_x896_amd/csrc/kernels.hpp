// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias,
                                float* logits, int T, int H, int E, hipStream_t stream);
hipError_t launch_router_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                              hipStream_t stream);
hipError_t launch_plan(const int32_t* ids, int n_pairs, int E, Plan plan, hipStream_t stream);

// Everything the decode-path expert kernels need.
struct GemvLayer {
  int T, H, I, E, k, S;
  const uint16_t* x;        // bf16 [T][H]
  const uint8_t* experts;   // E records
  uint64_t stride;          // bytes between records
  const uint16_t* sgate;    // bf16 [S][I][H]
  const uint16_t* sup;      // bf16 [S][I][H]
  const uint16_t* sdown;    // bf16 [S][H][I]
  Plan plan;
  int max_active;           // upper bound on plan.n_active (grid sizing)
  float* h;                 // fp32 [T*k][I]   routed SiLU(g)*u per pair
  float* hs;                // fp32 [S][T][I]  shared SiLU(g)*u
  float* part;              // fp32 [T*k][H]   routed expert outputs per pair
  float* ysh;               // fp32 [T][H]     sum of shared expert outputs
};

hipError_t launch_gateup(const GemvLayer& L, hipStream_t stream);
hipError_t launch_down(const GemvLayer& L, hipStream_t stream);
hipError_t launch_combine(const GemvLayer& L, const float* w,
                          const uint16_t* residual, uint16_t* y, hipStream_t stream);

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H,
                          uint16_t* out, hipStream_t stream);
hipError_t launch_dequant_export(const uint8_t* record, int H, int I, int matrix, float* out,
                                 hipStream_t stream);
hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int K, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);

}  // namespace moe
