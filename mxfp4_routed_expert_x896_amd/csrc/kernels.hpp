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
// Largest T for which one workgroup selects all tokens and builds the plan.
constexpr int kSelectPlanMaxTokens = 64;
hipError_t launch_router_select_plan(const float* logits, int T, int E, int k, int32_t* ids,
                                     float* w, Plan plan, int* zero, int n_zero,
                                     hipStream_t stream);
// Also zeroes n_zero ints at zero (the down kernel's tile counters).
hipError_t launch_plan(const int32_t* ids, int n_pairs, int E, Plan plan, int* zero, int n_zero,
                       hipStream_t stream);

// Everything the decode-path expert kernels need.
struct GemvLayer {
  int T, H, I, E, k, S;
  const uint16_t* x;        // bf16 [T][H]
  const uint8_t* experts;   // E packed records (MFMA-tiled, see pack.hip)
  uint64_t stride;          // bytes between records
  const uint16_t* sgate;    // bf16 [S] packed [I][H]
  const uint16_t* sup;      // bf16 [S] packed [I][H]
  const uint16_t* sdown;    // bf16 [S] packed [H][I]
  Plan plan;
  int max_active;           // upper bound on plan.n_active (grid sizing)
  int mtp_gu, mtp_d;        // tokens staged per LDS pass (set by the launchers)
  uint16_t* h;              // bf16 [2][T*k][I] routed SiLU(g)*u per pair, hi and lo parts
  uint16_t* hs;             // bf16 [2][S][T][I] shared SiLU(g)*u, hi and lo parts
  float* part;              // fp32 [T*k][H]   routed expert outputs per pair
  float* ysh;               // fp32 [S][T][H]  shared expert outputs
  int* tile_cnt;            // [ceil(H / 64)] arrivals per down tile (zeroed by the plan kernel)
  const float* w;           // fp32 [T][k] combine weights
  const uint16_t* residual; // bf16 [T][H] or null
  uint16_t* y;              // bf16 [T][H]
};

hipError_t launch_gateup(GemvLayer L, hipStream_t stream);
hipError_t launch_down(GemvLayer L, hipStream_t stream);

// Repacking (pack.hip).
size_t packed_mxfp4_bytes(int R, int K);
size_t packed_record_bytes(int H, int I);
hipError_t launch_pack_record(const uint8_t* src, int H, int I, uint8_t* dst, hipStream_t stream);
hipError_t launch_pack_bf16(const uint16_t* src, int R, int K, uint16_t* dst, hipStream_t stream);

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H,
                          uint16_t* out, hipStream_t stream);
hipError_t launch_dequant_export(const uint8_t* record, int H, int I, int matrix, float* out,
                                 hipStream_t stream);
hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int K, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);

}  // namespace moe
