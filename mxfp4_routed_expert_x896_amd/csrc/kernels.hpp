// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

// Timing hook: the pair of events the next kernel launch stamps with its own
// start and end (both null when the calling thread registered none).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents next_launch_events();  // api.hip

// A launch that stamps ev when the hook is active: the dispatch itself takes
// the timestamps, so the pair spans exactly the kernel's execution.
template <typename K, typename... A>
inline void launch_timed(LaunchEvents ev, K kernel, dim3 grid, dim3 block, uint32_t lds,
                         hipStream_t stream, A... args) {
  if (ev.start != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev.start, ev.stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
}

// Value of the workspace status word after a top-k wait gave up (even, so
// never an epoch; any other value means no wait gave up).
constexpr unsigned long long kWaitGaveUp = 0x5449'4D45'4F55'5400ull;
// Default number of polls before a top-k wait gives up (~0.3 us each).
constexpr long kDefaultSpinLimit = 1l << 20;

// Tokens per pass of the GEMV path's shared-expert roles: the 16 B columns
// of one MFMA (the shared down's pass takes 8, each token's h as two
// columns, hi and lo).
constexpr int kGemvPassTokens = 16;
// Output rows per routed down workgroup (and per combine tile).
constexpr int kDownRows = 128;
static_assert(kDownRows % 16 == 0, "whole row groups");
// Routed down rows per workgroup when the down runs in the one-token front
// launch (half as many workgroups, each wave streams twice as long).
constexpr int kFrontDownRows = 256;
static_assert(kFrontDownRows % kDownRows == 0, "front tiles count on the same counters");
// Tokens whose top-k and plan run in the router launch, on one workgroup
// (its waves take the tokens in turn) that waits for the logits.
constexpr int kSelwMaxTokens = 8;
// Router logits of kRouterSplitMin or more tokens on the GEMV path: bf16
// MFMA over kRouterSplit quarters of the contraction, one workgroup per
// (16 experts, quarter), partial sums added in order by the top-k.
constexpr int kRouterSplit = 4;
constexpr int kRouterSplitMin = 5;
// Prefill combine workgroups per token: 1024-column chunks of the output row.
__host__ __device__ inline int combine_chunks(int H) { return (H + 1023) / 1024; }
// Consecutive prefill token tiles that one XCD runs side by side.
constexpr int kMxGroup = 4;
// Threads of a prefill routed-expert GEMM workgroup (8 waves; the other
// launches use 4).
constexpr int kMxThreads = 512;
// Weight rows per prefill routed GEMM workgroup: gate/up takes 256 rows of
// the intermediate dimension (of both matrices), down 512 rows of hidden.
constexpr int kMxRowsGU = 256;
constexpr int kMxRowsD = 512;

// Everything the layer kernels need (layer.hip).
struct GemvLayer {
  int T, H, I, E, k, S;
  const uint16_t* x;        // bf16 [T][H]
  const uint16_t* wr;       // bf16 [E][H] router weights
  const float* rbias;       // fp32 [E] bias added to the logits, or null
  const float* sbias;       // fp32 [E] bias added to the scores for the choice only, or null
  float rscale;             // factor on the combine weights
  float* logits;            // fp32 [T][E]
  const int32_t* ids_in;    // int32 [T][k] routing given by the caller (plan role), or
                            // written by the top-k role of an earlier launch (direct mode)
  int32_t* ids_out;         // int32 [T][k] routing written by the top-k role
  float* w_out;             // fp32 [T][k] weights written by the top-k role
  int* sel_cnt;             // [1] arrivals of top-k workgroups (zeroed by the logits launch)
  const uint8_t* experts;   // E packed records (MFMA-tiled, see pack.hip), or a pool
  const int32_t* eslot;     // pool: expert -> record index (clamped to n_slots), else NULL
  int n_slots;
  uint64_t stride;          // bytes between records
  const uint16_t* sgate;    // bf16 [S] packed [I][H]
  const uint16_t* sup;      // bf16 [S] packed [I][H]
  const uint16_t* sdown;    // bf16 [S] packed [H][I]
  Plan plan;
  // Direct mode (one token): expert slot a is pair a, its expert ids_in[a];
  // no plan is built (the k experts of one token are distinct).
  int direct;
  // Completion flags of the logits workgroups ([n_logits], near the start
  // of the workspace): each stores `epoch` once its logits are stored, for a
  // top-k workgroup of the same launch to wait on; that workgroup clears
  // them.  epoch differs between calls (odd values).  A wait that gives up
  // after spin_limit polls stores kWaitGaveUp into *status (the first word
  // of the workspace), which only moe_workspace_status clears.
  unsigned long long* lflags;
  unsigned long long* status;
  unsigned long long epoch;
  long spin_limit;
  // 1: logits[t][e] complete; kRouterSplit: logits holds kRouterSplit partial
  // sums [q][t][e] over quarters of the contraction (bias in quarter 0),
  // which the top-k adds in order
  int lsplit;
  int n_tiles;              // ceil(H / kDownRows) routed down tiles (set by the launcher)
  int n_stiles;             // ceil(H / 64) shared down tiles (set by the launcher)
  int mtp_gu, mtp_d;        // tokens staged per LDS pass (set by the launcher)
  uint32_t* h;              // [T*k][I] routed SiLU(g)*u in plan slot order (row p for
                            // pairs[p]): bf16 hi | bf16 lo << 16
  uint16_t* hs;             // bf16 [2][S][T][I] shared SiLU(g)*u, hi and lo parts
  float* part;              // fp32 [T*k][H]   routed expert outputs per pair
  float* ysh;               // fp32 [S][T][H]  shared expert outputs
  int* tile_cnt;            // [n_tiles] routed down arrivals per output tile (zeroed by
                            // the plan builder, for one token the top-k, of the call)
  // One-token decode (moe_decode_front: the whole layer in one launch).
  // The top-k, once its ids, weights and cleared arrival counters are
  // stored, stores idtag[a] = (epoch mod 2^48) << 16 | expert of slot a
  // (E <= 1024), which a routed workgroup of slot a polls for both its
  // go-ahead and its expert, and `epoch` into *idsflag, which the shared down
  // workgroups wait for before they count arrivals.  Each shared gate/up
  // workgroup stores `epoch` into sgflags[sx * I/16 + rg] once its h rows are
  // stored (the shared down of expert sx waits for them); each routed gate/up
  // workgroup into guflags[a * I/32 + tile] (the routed down of slot a waits
  // for them).  The routed down runs on kFrontDownRows-row tiles; the shared
  // down workgroups count on the tiles' arrival counters beside the routed
  // down ones, and whichever arrives last combines the tile.
  int front;
  unsigned long long* idsflag;
  unsigned long long* sgflags;
  unsigned long long* guflags;
  unsigned long long* idtag;
  // prefill (MFMA) path: MX activations, rows padded to Kq / Iq columns
  // (multiples of 512, zero codes past H / I); scale rows in MFMA order.
  // afmt 0: MXFP8 (E4M3, one byte per element); afmt 4: MXFP4 (E2M1, two per
  // byte, even element in the low nibble: rows of Kq / 2 and Iq / 2 bytes)
  int Kq, Iq;
  int afmt;
  uint8_t* xq;              // codes [T][Kq] (FP8) or [T][Kq / 2] (FP4)
  uint8_t* xs;              // E8M0 [T][Kq / 32]
  uint8_t* hq;              // codes [T*k][Iq] or [T*k][Iq / 2]: routed SiLU(g)*u per pair
  uint8_t* hs8;             // E8M0 [T*k][Iq / 32]
  const float* w;           // fp32 [T][k] combine weights
  const uint16_t* residual; // bf16 [T][H] or null
  uint16_t* y;              // bf16 [T][H]
};

// Workgroups of each role in one launch (0 = role absent).
struct Stage {
  int n_logits = 0;           // ceil(E / 4)
  int n_select = 0;           // ceil(T / 4)
  int n_selw = 0;             // 0 or 1: top-k (T <= 8) after waiting for this launch's logits
  int plan_after_select = 0;  // the last top-k workgroup builds the plan
  int n_plan = 0;             // 0 or 1
  int n_sgu = 0;              // S * I / 16 (x passes of 16 tokens, XCD-grouped; the front: one)
  int n_sdn = 0;              // S * ceil(H / 64) (x passes of 8 tokens, XCD-grouped; the front: one)
  int n_rgu = 0;              // max_active * I / 32
  int n_rdn = 0;              // max_active * ceil(H / kDownRows)
  int n_xq = 0;               // x quantisation, 256 blocks of 32 per workgroup
  int n_mgu = 0;              // max token tiles * ceil(I / 128)  (prefill gate/up)
  int n_mdn = 0;              // max token tiles * ceil(H / 256)  (prefill down)
  int n_comb = 0;             // T  (prefill combine, one token per workgroup)
  int n_rmx = 0;              // ceil(E / 256) * ceil(T / 64)  (prefill router)
  int n_sgmx = 0;             // XCD-ordered grid over (S x ceil(I / 128), ceil(T / 64))
  int n_sdmx = 0;             // XCD-ordered grid over (S x ceil(H / 256), ceil(T / 64))
};

enum class StageKind {
  RouterSharedGateUp,  // roles: logits, shared gate/up, top-k waiting for the logits
  DecodeFront,         // one token, the whole layer: logits, shared gate/up, top-k, routed
                       // gate/up and down, shared down, combine; roles wait on flags of
                       // blocks before them
  SelectSharedDown,    // roles: top-k (+ plan), shared down
  PlanSharedGateUp,    // roles: plan, shared gate/up
  RoutedGateUp,        // roles: shared down, routed gate/up
  RoutedDownCombine,   // roles: routed down + combine
  PlanQuantSharedGateUp,  // plan, x -> MXFP8 (prefill), shared gate/up (decode)
  RouterMxQuant,       // prefill: x -> MXFP8, router logits (MFMA)
  MxGateUp,            // prefill (8-wave workgroups): routed gate/up (scaled MFMA), shared
                       // gate/up (bf16 MFMA)
  MxDown,              // prefill (8-wave workgroups): routed down -> per-pair partials,
                       // shared down
  Combine,             // prefill: weighted combine of the partials
};

hipError_t launch_stage(StageKind kind, GemvLayer L, Stage st, hipStream_t stream);

// Repacking (pack.hip).
size_t packed_mxfp4_bytes(int R, int K);
size_t packed_record_bytes(int H, int I);
hipError_t launch_pack_record(const uint8_t* src, int H, int I, uint8_t* dst, hipStream_t stream);
hipError_t launch_pack_bf16(const uint16_t* src, int R, int K, uint16_t* dst, hipStream_t stream);

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H,
                          uint16_t* out, hipStream_t stream);
hipError_t launch_dequant_export(const uint8_t* record, int H, int I, int matrix, float* out,
                                 hipStream_t stream);
// Row-scaled int8 -> fp32 (spine.hip); blocks the launch uses (< 2^32 required).
int64_t int8_dequant_blocks(int64_t rows, int64_t cols);
hipError_t launch_int8_row_dequant(const int8_t* q, const float* scale, int64_t rows, int64_t cols,
                                   float* out, hipStream_t stream);
// Block-scaled 16x16x128 MFMA issue rate (rate.hip): formats 4 = FP4 E2M1,
// 0 = FP8 E4M3; supported pairs (4, 4), (4, 0), (0, 0).
hipError_t launch_mfma_rate(int a_fmt, int b_fmt, int64_t iters, int blocks, float* out,
                            hipStream_t stream);
hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int K, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);

}  // namespace moe
