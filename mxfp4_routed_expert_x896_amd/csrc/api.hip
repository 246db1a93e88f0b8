// C ABI of the MoE layer library: host-side validation, workspace carving
// and launch sequencing on the caller's stream.  See include/moe_mxfp4.h.
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <climits>
#include <cstring>
#include <mutex>

#include "../../include/moe_mxfp4.h"
#include "common.hpp"
#include "kernels.hpp"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip_error = 0;

// Benchmark timing hook (see moe_profile_events in the header).
struct ProfileHook {
  hipEvent_t* events = nullptr;
  int n = 0;
  int used = 0;
};
thread_local ProfileHook g_prof;

// Polls before a top-k wait gives up (moe_set_wait_limit), per host thread.
thread_local long g_wait_limit = moe::kDefaultSpinLimit;

// Each call that launches timed kernels starts a new sequence of event pairs.
void prof_begin(hipStream_t) { g_prof.used = 0; }

}  // namespace

moe::LaunchEvents moe::next_launch_events() {
  LaunchEvents ev;
  if (g_prof.events != nullptr && g_prof.used + 2 <= g_prof.n) {
    ev.start = g_prof.events[g_prof.used];
    ev.stop = g_prof.events[g_prof.used + 1];
    g_prof.used += 2;
  }
  return ev;
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return MOE_EDEVICE;
  int st = g_device_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_EDEVICE;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MOE_OK : MOE_EDEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launched(hipError_t e, hipStream_t) {
  if (e != hipSuccess) {
    g_last_hip_error = int(e);
    return MOE_ELAUNCH;
  }
  return MOE_OK;
}

uint64_t record_bytes(int H, int I) {
  return 3ull * (uint64_t(H) * I / 2 + uint64_t(H) * I / 32);
}

int check_layer(const moe_layer_desc* L) {
  if (L == nullptr) return MOE_EINVAL;
  if (L->hidden <= 0 || L->inter <= 0 || L->n_experts <= 0 || L->top_k <= 0 || L->n_shared < 0)
    return MOE_EINVAL;
  if (L->router_mode != MOE_ROUTER_BIAS_LOGITS && L->router_mode != MOE_ROUTER_BIAS_SELECT)
    return MOE_EINVAL;
  if (!(L->routed_scale >= 0.0f && L->routed_scale <= 3.0e38f)) return MOE_EINVAL;  // NaN, inf
  if (L->expert_slot == nullptr ? L->n_slots != 0 : L->n_slots <= 0) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(L->expert_slot) & 3u) return MOE_EALIGN;
  if (L->hidden % 32 || L->inter % 32 || L->hidden > 8192 || L->inter > 8192) return MOE_ESHAPE;
  if (L->n_experts > 1024 || L->top_k > 32 || L->top_k > L->n_experts || L->n_shared > 4)
    return MOE_ESHAPE;
  if (L->router_w == nullptr || L->experts == nullptr) return MOE_EINVAL;
  if (L->n_shared > 0 &&
      (L->shared_gate == nullptr || L->shared_up == nullptr || L->shared_down == nullptr))
    return MOE_EINVAL;
  if (!aligned16(L->router_w) || !aligned16(L->experts) || (L->expert_stride & 15u))
    return MOE_EALIGN;
  if (L->router_bias != nullptr && !aligned16(L->router_bias)) return MOE_EALIGN;
  if (L->n_shared > 0 &&
      (!aligned16(L->shared_gate) || !aligned16(L->shared_up) || !aligned16(L->shared_down)))
    return MOE_EALIGN;
  if (L->expert_stride < moe::packed_record_bytes(L->hidden, L->inter)) return MOE_ESHAPE;
  return MOE_OK;
}

constexpr int64_t kMaxTokens = 1 << 16;
// MOE_PATH_AUTO switches to the MFMA (prefill) path from this many tokens.
constexpr int64_t kMfmaMinTokens = 256;

uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

int n_tiles(const moe_layer_desc* L) { return (L->hidden + moe::kDownRows - 1) / moe::kDownRows; }
uint64_t pad512(uint64_t v) { return (v + 511) / 512 * 512; }
// Upper bound on the prefill token tiles (kPlanTileTokens pairs of one expert each).
int max_mtiles(const moe_layer_desc* L, int64_t T) {
  const int64_t pairs = T * L->top_k;
  const int64_t active = pairs < L->n_experts ? pairs : L->n_experts;
  return int((pairs + (moe::kPlanTileTokens - 1) * active) / moe::kPlanTileTokens + 1);
}
int n_shared_tiles(const moe_layer_desc* L) { return (L->hidden + 63) / 64; }
// Workgroups of the GEMV launches' shared roles for T tokens: (expert, row
// group or 64-row tile, pass of tokens), grouped by XCD (layer.hip
// xcd_split: 8 units per group of blocks, the passes of a unit on one XCD).
int xcd_units(int units, int passes) { return 8 * ((units + 7) / 8) * passes; }
int n_sgu_wgs(const moe_layer_desc* L, int64_t T) {
  const int pass = moe::kGemvPassTokens;
  return xcd_units(L->n_shared * (L->inter / 16), int((T + pass - 1) / pass));
}
int n_sdn_wgs(const moe_layer_desc* L, int64_t T) {
  const int pass = moe::kGemvPassTokens / 2;
  return xcd_units(L->n_shared * n_shared_tiles(L), int((T + pass - 1) / pass));
}

int n_logit_wgs(const moe_layer_desc* L) { return (L->n_experts + 3) / 4; }
// Router workgroups of the GEMV path for T tokens (see lsplit).
int router_split(int64_t T) { return T >= moe::kRouterSplitMin ? moe::kRouterSplit : 1; }
int n_router_wgs(const moe_layer_desc* L, int64_t T) {
  return router_split(T) > 1 ? (L->n_experts + 15) / 16 * moe::kRouterSplit : n_logit_wgs(L);
}

// A value no earlier call stored in the logits flags: odd numbers from a
// per-process start, so it is never 0 (the cleared state).
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> ctr{
      (uint64_t(std::chrono::steady_clock::now().time_since_epoch().count()) << 20) |
      (uint64_t(getpid()) & 0xFFFFF)};
  return ctr.fetch_add(2, std::memory_order_relaxed) | 1ull;
}

// Workspace layout for T tokens.
struct Carve {
  uint64_t status, lflags, idsflag, sgflags, guflags, idtag, logits, n_active, active, act_off, pairs, h, hs, part, ysh, tile_cnt, sel_cnt;
  uint64_t n_mtiles, mtiles, xq, xs, hq, hs8, total;
};

Carve carve(const moe_layer_desc* L, int64_t T) {
  const uint64_t E = L->n_experts, k = L->top_k, H = L->hidden, I = L->inter, S = L->n_shared;
  const uint64_t t = uint64_t(T);
  Carve c;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = align256(off + bytes);
    return at;
  };
  c.status = take(8);  // first: the same place for every layer and T
  // flags of the logits workgroups (either router decomposition)
  c.lflags = take(uint64_t(std::max(n_logit_wgs(L), (L->n_experts + 15) / 16 * moe::kRouterSplit)) * 8);
  c.idsflag = take(8);
  c.sgflags = take(S * (I / 16) * 8);
  c.guflags = take((T == 1 ? k * (I / 32) : 1) * 8);  // one token: routed gate/up flags
  c.idtag = take(k * 8);
  c.logits = take(t * E * 4 * (T >= moe::kRouterSplitMin ? moe::kRouterSplit : 1));
  c.n_active = take(4);
  c.active = take(E * 4);
  c.act_off = take((E + 1) * 4);
  c.pairs = take(t * k * 4);
  c.h = take(t * k * I * 4);
  c.hs = take(S * t * I * 4);
  c.part = take(t * k * H * 4);
  c.ysh = take(S * t * H * 4);
  c.tile_cnt = take(n_tiles(L) * 4);
  c.sel_cnt = take(4);
  const uint64_t Kq = pad512(H), Iq = pad512(I);
  c.n_mtiles = take(4);
  c.mtiles = take(uint64_t(max_mtiles(L, T)) * 4);
  c.xq = take(t * Kq);
  c.xs = take(t * Kq / 32);
  c.hq = take(t * k * Iq);
  c.hs8 = take(t * k * Iq / 32);
  c.total = off;
  return c;
}

template <typename T>
T* at(void* ws, uint64_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

int check_tokens(int64_t T) {
  if (T <= 0) return MOE_EINVAL;
  if (T > kMaxTokens) return MOE_ESHAPE;
  return MOE_OK;
}

int check_ws(const moe_layer_desc* L, int64_t T, void* ws, uint64_t ws_bytes) {
  if (ws == nullptr) return MOE_EINVAL;
  if (!aligned16(ws)) return MOE_EALIGN;
  if (ws_bytes < carve(L, T).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

moe::GemvLayer gemv_layer(const moe_layer_desc* L, const uint16_t* x, int64_t T, void* ws) {
  const Carve c = carve(L, T);
  moe::GemvLayer G = {};
  G.T = int(T);
  G.H = L->hidden;
  G.I = L->inter;
  G.E = L->n_experts;
  G.k = L->top_k;
  G.S = L->n_shared;
  G.x = x;
  G.wr = L->router_w;
  G.rbias = L->router_mode == MOE_ROUTER_BIAS_LOGITS ? L->router_bias : nullptr;
  G.sbias = L->router_mode == MOE_ROUTER_BIAS_SELECT ? L->router_bias : nullptr;
  G.rscale = L->routed_scale == 0.0f ? 1.0f : L->routed_scale;
  G.logits = at<float>(ws, c.logits);
  G.lflags = at<unsigned long long>(ws, c.lflags);
  G.status = at<unsigned long long>(ws, c.status);
  G.idsflag = at<unsigned long long>(ws, c.idsflag);
  G.sgflags = at<unsigned long long>(ws, c.sgflags);
  G.guflags = at<unsigned long long>(ws, c.guflags);
  G.idtag = at<unsigned long long>(ws, c.idtag);
  G.epoch = next_epoch();
  G.spin_limit = g_wait_limit;
  G.lsplit = 1;
  G.sel_cnt = at<int>(ws, c.sel_cnt);
  G.experts = L->experts;
  G.stride = L->expert_stride;
  G.eslot = L->expert_slot;
  G.n_slots = L->n_slots;
  G.sgate = L->shared_gate;
  G.sup = L->shared_up;
  G.sdown = L->shared_down;
  G.plan.n_active = at<int32_t>(ws, c.n_active);
  G.plan.active = at<int32_t>(ws, c.active);
  G.plan.act_off = at<int32_t>(ws, c.act_off);
  G.plan.pairs = at<int32_t>(ws, c.pairs);
  G.h = at<uint32_t>(ws, c.h);
  G.hs = at<uint16_t>(ws, c.hs);
  G.part = at<float>(ws, c.part);
  G.ysh = at<float>(ws, c.ysh);
  G.tile_cnt = at<int>(ws, c.tile_cnt);
  G.plan.n_mtiles = at<int32_t>(ws, c.n_mtiles);
  G.plan.mtiles = at<int32_t>(ws, c.mtiles);
  G.Kq = int(pad512(L->hidden));
  G.Iq = int(pad512(L->inter));
  G.xq = at<uint8_t>(ws, c.xq);
  G.xs = at<uint8_t>(ws, c.xs);
  G.hq = at<uint8_t>(ws, c.hq);
  G.hs8 = at<uint8_t>(ws, c.hs8);
  return G;
}

// Workgroup counts of the roles (see layer.hip).
int n_select_wgs(int64_t T) { return int((T + 3) / 4); }
int max_active(const moe_layer_desc* L, int64_t T) {
  const int64_t pairs = T * L->top_k;
  return int(pairs < L->n_experts ? pairs : L->n_experts);
}

int stage(moe::StageKind kind, const moe::GemvLayer& G, const moe::Stage& st,
          hipStream_t stream) {
  return launched(moe::launch_stage(kind, G, st, stream), stream);
}

// Router only: logits, then the top-k.
int do_route(const moe_layer_desc* L, const uint16_t* x, int64_t T, int32_t* ids, float* w,
             void* ws, hipStream_t stream) {
  moe::GemvLayer G = gemv_layer(L, x, T, ws);
  G.ids_out = ids;
  G.w_out = w;
  G.lsplit = router_split(T);
  moe::Stage s1;
  s1.n_logits = n_router_wgs(L, T);
  int st = stage(moe::StageKind::RouterSharedGateUp, G, s1, stream);
  if (st) return st;
  moe::Stage s2;
  s2.n_select = n_select_wgs(T);
  return stage(moe::StageKind::SelectSharedDown, G, s2, stream);
}

// Given routing: plan + shared gate/up, shared down + routed gate/up,
// routed down + combine.
int do_forward_gemv(const moe_layer_desc* L, const uint16_t* x, int64_t T, const int32_t* ids,
                    const float* w, const uint16_t* residual, uint16_t* y, void* ws,
                    hipStream_t stream) {
  moe::GemvLayer G = gemv_layer(L, x, T, ws);
  G.ids_in = ids;
  G.direct = T == 1;
  G.w = w;
  G.residual = residual;
  G.y = y;
  const int S = L->n_shared, tiles_gu = L->inter / 32, ma = max_active(L, T);
  moe::Stage s1;
  s1.n_plan = 1;
  s1.n_sgu = n_sgu_wgs(L, T);
  int st = stage(moe::StageKind::PlanSharedGateUp, G, s1, stream);
  if (st) return st;
  moe::Stage s2;
  s2.n_sdn = n_sdn_wgs(L, T);
  s2.n_rgu = ma * tiles_gu;
  if ((st = stage(moe::StageKind::RoutedGateUp, G, s2, stream))) return st;
  moe::Stage s3;
  s3.n_rdn = ma * n_tiles(L);
  return stage(moe::StageKind::RoutedDownCombine, G, s3, stream);
}

// Given routing, with the routed experts' records arriving on another
// stream (expert pool): the shared experts first -- plan + shared gate/up,
// shared down -- then the stream waits for `ready` (recorded by the caller
// after the records' copies), then routed gate/up and routed down + combine.
// The shared experts' weight stream overlaps the copies.
int do_forward_gemv_after(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                          const int32_t* ids, const float* w, const uint16_t* residual,
                          uint16_t* y, void* ws, hipEvent_t ready, hipStream_t stream) {
  moe::GemvLayer G = gemv_layer(L, x, T, ws);
  G.ids_in = ids;
  G.direct = T == 1;
  G.w = w;
  G.residual = residual;
  G.y = y;
  const int S = L->n_shared, tiles_gu = L->inter / 32, ma = max_active(L, T);
  moe::Stage s1;
  s1.n_plan = 1;
  s1.n_sgu = n_sgu_wgs(L, T);
  int st = stage(moe::StageKind::PlanSharedGateUp, G, s1, stream);
  if (st) return st;
  if (S > 0) {
    moe::Stage s1b;  // the shared down alone (the routed gate/up launch without its routed part)
    s1b.n_sdn = n_sdn_wgs(L, T);
    if ((st = stage(moe::StageKind::RoutedGateUp, G, s1b, stream))) return st;
  }
  if ((st = launched(hipStreamWaitEvent(stream, ready, 0), stream))) return st;
  moe::Stage s2;
  s2.n_rgu = ma * tiles_gu;
  if ((st = stage(moe::StageKind::RoutedGateUp, G, s2, stream))) return st;
  moe::Stage s3;
  s3.n_rdn = ma * n_tiles(L);
  return stage(moe::StageKind::RoutedDownCombine, G, s3, stream);
}

// Router and experts: logits + shared gate/up, top-k + plan + shared down,
// routed gate/up, routed down + combine.
int do_layer_gemv(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                  const uint16_t* residual, uint16_t* y, int32_t* ids, float* w, void* ws,
                  hipStream_t stream) {
  moe::GemvLayer G = gemv_layer(L, x, T, ws);
  G.ids_out = ids;
  G.ids_in = ids;  // read back by the routed down launch in direct mode
  G.w_out = w;
  G.w = w;
  G.residual = residual;
  G.y = y;
  G.lsplit = router_split(T);
  const int S = L->n_shared, tiles_gu = L->inter / 32, ma = max_active(L, T);
  moe::Stage s1;
  s1.n_logits = n_router_wgs(L, T);
  s1.n_sgu = n_sgu_wgs(L, T);
  if (T == 1) {
    // one token: the whole layer in one launch whose workgroups wait on
    // flags of earlier blocks (moe_decode_front); no plan (direct mode)
    G.direct = 1;
    G.front = 1;
    s1.n_selw = 1;
    s1.plan_after_select = 1;
    // the front's own decomposition: one workgroup per shared row group / tile
    s1.n_sgu = S * (L->inter / 16);
    s1.n_rgu = ma * tiles_gu;
    s1.n_sdn = S * n_shared_tiles(L);
    s1.n_rdn = ma * ((L->hidden + moe::kFrontDownRows - 1) / moe::kFrontDownRows);
    return stage(moe::StageKind::DecodeFront, G, s1, stream);
  }
  if (T <= moe::kSelwMaxTokens) {
    // 2 to kSelwMaxTokens tokens: the top-k and the plan run in the router
    // launch, on one workgroup that waits for the logits
    s1.n_selw = 1;
    s1.plan_after_select = 1;
    int st = stage(moe::StageKind::RouterSharedGateUp, G, s1, stream);
    if (st) return st;
    moe::Stage s3;
    s3.n_rgu = ma * tiles_gu;
    s3.n_sdn = n_sdn_wgs(L, T);
    if ((st = stage(moe::StageKind::RoutedGateUp, G, s3, stream))) return st;
    moe::Stage s4;
    s4.n_rdn = ma * n_tiles(L);
    return stage(moe::StageKind::RoutedDownCombine, G, s4, stream);
  }
  int st = stage(moe::StageKind::RouterSharedGateUp, G, s1, stream);
  if (st) return st;
  moe::Stage s2;
  s2.n_select = n_select_wgs(T);
  s2.plan_after_select = 1;
  s2.n_sdn = n_sdn_wgs(L, T);
  if ((st = stage(moe::StageKind::SelectSharedDown, G, s2, stream))) return st;
  moe::Stage s3;
  s3.n_rgu = ma * tiles_gu;
  if ((st = stage(moe::StageKind::RoutedGateUp, G, s3, stream))) return st;
  moe::Stage s4;
  s4.n_rdn = ma * n_tiles(L);
  return stage(moe::StageKind::RoutedDownCombine, G, s4, stream);
}

int n_quant_wgs(const moe::GemvLayer& G, int64_t T) { return int((T * (G.Kq / 32) + 255) / 256); }
int n_token_tiles(int64_t T) { return int((T + 63) / 64); }
// Grid of an XCD-ordered role over (pairs, token tiles): see xcd_split.
int xcd_grid(int n_pairs, int64_t T) { return 8 * ((n_pairs + 7) / 8) * n_token_tiles(T); }
// Grid of the prefill shared-expert role, two token tiles per workgroup
// (see shared_mx_unit).
int shared_mx_grid(int n_pairs, int64_t T) {
  return 8 * ((n_pairs + 7) / 8) * ((n_token_tiles(T) + 1) / 2);
}

// Prefill experts once the plan and the MXFP8 x exist: routed gate/up
// (scaled MFMA) + shared gate/up (bf16 MFMA); routed down -> per-pair
// partials + shared down; combine.  The GEMM launches run 8-wave
// workgroups; the routed roles' blocks come first, so the shared tiles fill
// the tail.
// Blocks of a prefill GEMM launch over mt token tiles and tiles_r row tiles:
// the XCD-grouped order of the launch (kMxGroup token tiles per XCD visit)
// needs whole rounds of 8 groups.
int mx_blocks(int mt, int tiles_r) {
  const int round = 8 * moe::kMxGroup;
  return round * ((mt + round - 1) / round) * tiles_r;
}

int mfma_experts(const moe_layer_desc* L, const moe::GemvLayer& G, int64_t T, hipStream_t stream) {
  const int S = L->n_shared, mt = max_mtiles(L, T);
  moe::Stage s2;
  s2.n_mgu = mx_blocks(mt, (L->inter + moe::kMxRowsGU - 1) / moe::kMxRowsGU);
  s2.n_sgmx = S > 0 ? shared_mx_grid(S * ((L->inter + 127) / 128), T) : 0;
  int st = stage(moe::StageKind::MxGateUp, G, s2, stream);
  if (st) return st;
  moe::Stage s3;
  s3.n_mdn = mx_blocks(mt, (L->hidden + moe::kMxRowsD - 1) / moe::kMxRowsD);
  s3.n_sdmx = S > 0 ? shared_mx_grid(S * ((L->hidden + 255) / 256), T) : 0;
  if ((st = stage(moe::StageKind::MxDown, G, s3, stream))) return st;
  moe::Stage s4;
  s4.n_comb = int(T) * moe::combine_chunks(L->hidden);
  return stage(moe::StageKind::Combine, G, s4, stream);
}

// Prefill layer: x -> MXFP8 + router logits (MFMA); top-k + plan; experts.
int do_layer_mfma(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                  const uint16_t* residual, uint16_t* y, int32_t* ids, float* w, void* ws,
                  int afmt, hipStream_t stream) {
  moe::GemvLayer G = gemv_layer(L, x, T, ws);
  G.afmt = afmt;
  G.ids_out = ids;
  G.w_out = w;
  G.w = w;
  G.residual = residual;
  G.y = y;
  moe::Stage s0;
  s0.n_xq = n_quant_wgs(G, T);
  s0.n_rmx = ((L->n_experts + 255) / 256) * n_token_tiles(T);
  int st = stage(moe::StageKind::RouterMxQuant, G, s0, stream);
  if (st) return st;
  moe::Stage s1;
  s1.n_select = n_select_wgs(T);
  s1.plan_after_select = 1;
  if ((st = stage(moe::StageKind::SelectSharedDown, G, s1, stream))) return st;
  return mfma_experts(L, G, T, stream);
}

// Prefill (MFMA) path for a given routing: plan + x -> MXFP8, then the
// experts.
int do_forward_mfma(const moe_layer_desc* L, const uint16_t* x, int64_t T, const int32_t* ids,
                    const float* w, const uint16_t* residual, uint16_t* y, void* ws, int afmt,
                    hipStream_t stream) {
  moe::GemvLayer G = gemv_layer(L, x, T, ws);
  G.afmt = afmt;
  G.ids_in = ids;
  G.w = w;
  G.residual = residual;
  G.y = y;
  moe::Stage s1;
  s1.n_plan = 1;
  s1.n_xq = n_quant_wgs(G, T);
  int st = stage(moe::StageKind::PlanQuantSharedGateUp, G, s1, stream);
  if (st) return st;
  return mfma_experts(L, G, T, stream);
}

int resolve_path(int32_t path, int64_t T) {
  if (path == MOE_PATH_AUTO) return T >= moe_mfma_min_tokens() ? MOE_PATH_MFMA : MOE_PATH_GEMV;
  return path;
}

bool valid_path(int32_t path) { return path >= MOE_PATH_AUTO && path <= MOE_PATH_MFMA_FP4; }
// MX activation format of an MFMA path (the MFMA's B-operand format code).
int act_format(int path) { return path == MOE_PATH_MFMA_FP4 ? 4 : 0; }

}  // namespace

MOE_API uint32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer or non-positive size)";
    case MOE_EALIGN: return "device pointer or stride not 16-byte aligned";
    case MOE_ESHAPE: return "unsupported shape";
    case MOE_EWORKSPACE: return "workspace smaller than moe_workspace_bytes()";
    case MOE_EDEVICE: return "current device is not gfx950";
    case MOE_ELAUNCH: return "kernel launch failed (see moe_last_hip_error)";
    case MOE_EUNSUPPORTED: return "request not implemented by the library";
    case MOE_ETIMEOUT: return "a top-k wait gave up: the routing of a call on this workspace is wrong";
    default: return "unknown status";
  }
}

MOE_API int moe_last_hip_error(void) { return g_last_hip_error; }

MOE_API int moe_profile_events(hipEvent_t* events, int32_t n_events) {
  if (events == nullptr || n_events <= 0) {
    g_prof = ProfileHook();
    return MOE_OK;
  }
  g_prof.events = events;
  g_prof.n = n_events;
  g_prof.used = 0;
  return MOE_OK;
}

MOE_API int moe_profile_count(void) { return g_prof.used; }

MOE_API int moe_record_bytes(int32_t hidden, int32_t inter, uint64_t* out_bytes) {
  if (out_bytes == nullptr || hidden <= 0 || inter <= 0) return MOE_EINVAL;
  if (hidden % 32 || inter % 32) return MOE_ESHAPE;
  *out_bytes = record_bytes(hidden, inter);
  return MOE_OK;
}

MOE_API int moe_packed_record_bytes(int32_t hidden, int32_t inter, uint64_t* out_bytes) {
  if (out_bytes == nullptr || hidden <= 0 || inter <= 0) return MOE_EINVAL;
  if (hidden % 32 || inter % 32) return MOE_ESHAPE;
  *out_bytes = moe::packed_record_bytes(hidden, inter);
  return MOE_OK;
}

MOE_API int moe_pack_experts(const uint8_t* src, uint64_t src_stride, uint8_t* dst,
                             uint64_t dst_stride, int32_t n_experts, int32_t hidden,
                             int32_t inter, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || n_experts <= 0 || hidden <= 0 || inter <= 0)
    return MOE_EINVAL;
  if (hidden % 32 || inter % 32 || hidden > 8192 || inter > 8192) return MOE_ESHAPE;
  if (src_stride < record_bytes(hidden, inter)) return MOE_ESHAPE;
  if (dst_stride < moe::packed_record_bytes(hidden, inter)) return MOE_ESHAPE;
  if (!aligned16(src) || !aligned16(dst) || (src_stride & 15u) || (dst_stride & 15u))
    return MOE_EALIGN;
  int st = check_device();
  if (st) return st;
  prof_begin(stream);
  for (int32_t e = 0; e < n_experts; ++e) {
    st = launched(moe::launch_pack_record(src + uint64_t(e) * src_stride, hidden, inter,
                                          dst + uint64_t(e) * dst_stride, stream),
                  stream);
    if (st) return st;
  }
  return MOE_OK;
}

MOE_API int moe_pack_bf16(const uint16_t* src, uint16_t* dst, int32_t count, int32_t rows,
                          int32_t cols, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || count <= 0 || rows <= 0 || cols <= 0) return MOE_EINVAL;
  if (rows % 16 || cols % 32) return MOE_ESHAPE;
  if (!aligned16(src) || !aligned16(dst)) return MOE_EALIGN;
  int st = check_device();
  if (st) return st;
  prof_begin(stream);
  const uint64_t n = uint64_t(rows) * cols;
  for (int32_t i = 0; i < count; ++i) {
    st = launched(moe::launch_pack_bf16(src + i * n, rows, cols, dst + i * n, stream), stream);
    if (st) return st;
  }
  return MOE_OK;
}

MOE_API int moe_workspace_bytes(const moe_layer_desc* layer, int64_t n_tokens,
                                uint64_t* out_bytes) {
  if (out_bytes == nullptr) return MOE_EINVAL;
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_tokens(n_tokens))) return st;
  *out_bytes = carve(layer, n_tokens).total;
  return MOE_OK;
}

MOE_API int64_t moe_mfma_min_tokens(void) { return kMfmaMinTokens; }

MOE_API int moe_route(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
                      int32_t* topk_ids, float* topk_w, void* workspace,
                      uint64_t workspace_bytes, hipStream_t stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_tokens(n_tokens))) return st;
  if (x == nullptr || topk_ids == nullptr || topk_w == nullptr) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w)) return MOE_EALIGN;
  if ((st = check_ws(layer, n_tokens, workspace, workspace_bytes))) return st;
  if ((st = check_device())) return st;
  prof_begin(stream);
  return do_route(layer, x, n_tokens, topk_ids, topk_w, workspace, stream);
}

MOE_API int moe_forward(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
                        const int32_t* topk_ids, const float* topk_w, const uint16_t* residual,
                        uint16_t* y, int32_t path, void* workspace, uint64_t workspace_bytes,
                        hipStream_t stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_tokens(n_tokens))) return st;
  if (x == nullptr || topk_ids == nullptr || topk_w == nullptr || y == nullptr) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(y))
    return MOE_EALIGN;
  if (residual != nullptr && !aligned16(residual)) return MOE_EALIGN;
  if (!valid_path(path)) return MOE_EINVAL;
  if ((st = check_ws(layer, n_tokens, workspace, workspace_bytes))) return st;
  if ((st = check_device())) return st;
  prof_begin(stream);
  const int p = resolve_path(path, n_tokens);
  if (p != MOE_PATH_GEMV)
    return do_forward_mfma(layer, x, n_tokens, topk_ids, topk_w, residual, y, workspace,
                           act_format(p), stream);
  return do_forward_gemv(layer, x, n_tokens, topk_ids, topk_w, residual, y, workspace, stream);
}

MOE_API int moe_forward_pooled(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
                               const int32_t* topk_ids, const float* topk_w,
                               const uint16_t* residual, uint16_t* y, int32_t path,
                               void* workspace, uint64_t workspace_bytes,
                               hipEvent_t records_ready, hipStream_t stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_tokens(n_tokens))) return st;
  if (x == nullptr || topk_ids == nullptr || topk_w == nullptr || y == nullptr) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(y))
    return MOE_EALIGN;
  if (residual != nullptr && !aligned16(residual)) return MOE_EALIGN;
  if (!valid_path(path)) return MOE_EINVAL;
  if ((st = check_ws(layer, n_tokens, workspace, workspace_bytes))) return st;
  if ((st = check_device())) return st;
  prof_begin(stream);
  const int p = resolve_path(path, n_tokens);
  if (p == MOE_PATH_GEMV && records_ready != nullptr)
    return do_forward_gemv_after(layer, x, n_tokens, topk_ids, topk_w, residual, y, workspace,
                                 records_ready, stream);
  // MFMA paths (their shared experts share the routed launches) or no event:
  // wait first, then the plain forward
  if (records_ready != nullptr &&
      (st = launched(hipStreamWaitEvent(stream, records_ready, 0), stream)))
    return st;
  if (p != MOE_PATH_GEMV)
    return do_forward_mfma(layer, x, n_tokens, topk_ids, topk_w, residual, y, workspace,
                           act_format(p), stream);
  return do_forward_gemv(layer, x, n_tokens, topk_ids, topk_w, residual, y, workspace, stream);
}

MOE_API int moe_layer(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
                      const uint16_t* residual, uint16_t* y, int32_t* topk_ids, float* topk_w,
                      int32_t path, void* workspace, uint64_t workspace_bytes,
                      hipStream_t stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_tokens(n_tokens))) return st;
  if (x == nullptr || topk_ids == nullptr || topk_w == nullptr || y == nullptr) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(y))
    return MOE_EALIGN;
  if (residual != nullptr && !aligned16(residual)) return MOE_EALIGN;
  if (!valid_path(path)) return MOE_EINVAL;
  if ((st = check_ws(layer, n_tokens, workspace, workspace_bytes))) return st;
  if ((st = check_device())) return st;
  prof_begin(stream);
  const int p = resolve_path(path, n_tokens);
  if (p != MOE_PATH_GEMV)
    return do_layer_mfma(layer, x, n_tokens, residual, y, topk_ids, topk_w, workspace,
                         act_format(p), stream);
  return do_layer_gemv(layer, x, n_tokens, residual, y, topk_ids, topk_w, workspace, stream);
}

// The workspace of moe_layer_scratch: one array per device, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address comes from hipGetSymbolAddress, once per
// device (scratch_address), and only that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[MOE_SCRATCH_BYTES];

namespace {

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array (looked up on the device's
// first call, with that device current).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EDEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      const int st = launched(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), nullptr);
      if (st) return st;
      if (p == nullptr) return MOE_ELAUNCH;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

MOE_API int moe_layer_scratch(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
                              const uint16_t* residual, uint16_t* y, int32_t* topk_ids,
                              float* topk_w, int32_t path, hipStream_t stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_tokens(n_tokens))) return st;
  if (x == nullptr || topk_ids == nullptr || topk_w == nullptr || y == nullptr) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(y))
    return MOE_EALIGN;
  if (residual != nullptr && !aligned16(residual)) return MOE_EALIGN;
  if (!valid_path(path)) return MOE_EINVAL;
  if (carve(layer, n_tokens).total > MOE_SCRATCH_BYTES) return MOE_EWORKSPACE;
  if ((st = check_device())) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  prof_begin(stream);
  const int p = resolve_path(path, n_tokens);
  if (p != MOE_PATH_GEMV)
    return do_layer_mfma(layer, x, n_tokens, residual, y, topk_ids, topk_w, ws, act_format(p),
                         stream);
  return do_layer_gemv(layer, x, n_tokens, residual, y, topk_ids, topk_w, ws, stream);
}

MOE_API int moe_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int64_t n_tokens,
                        int32_t hidden, uint16_t* out, hipStream_t stream) {
  if (x == nullptr || gamma == nullptr || out == nullptr || n_tokens <= 0 || hidden <= 0)
    return MOE_EINVAL;
  if (hidden % 32 || hidden > 8192 || n_tokens > INT_MAX) return MOE_ESHAPE;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(out)) return MOE_EALIGN;
  if (!(eps >= 0.0f)) return MOE_EINVAL;
  int st = check_device();
  if (st) return st;
  prof_begin(stream);
  return launched(moe::launch_rmsnorm(x, gamma, eps, int(n_tokens), hidden, out, stream), stream);
}

MOE_API int moe_dequant_export(const moe_layer_desc* layer, int32_t expert, int32_t matrix,
                               float* out, hipStream_t stream) {
  int st = check_layer(layer);
  if (st) return st;
  const int32_t n_rec = layer->expert_slot != nullptr ? layer->n_slots : layer->n_experts;
  if (out == nullptr || expert < 0 || expert >= n_rec || matrix < 0 || matrix > 2)
    return MOE_EINVAL;
  if (!aligned16(out)) return MOE_EALIGN;
  if ((st = check_device())) return st;
  const uint8_t* rec = layer->experts + uint64_t(expert) * layer->expert_stride;
  prof_begin(stream);
  return launched(
      moe::launch_dequant_export(rec, layer->hidden, layer->inter, matrix, out, stream), stream);
}

MOE_API int moe_int8_row_dequant(const int8_t* q, const float* scale, int64_t rows, int64_t cols,
                                 float* out, hipStream_t stream) {
  if (q == nullptr || scale == nullptr || out == nullptr || rows <= 0 || cols <= 0)
    return MOE_EINVAL;
  if (cols % 4) return MOE_ESHAPE;
  if ((reinterpret_cast<uintptr_t>(q) & 3u) || (reinterpret_cast<uintptr_t>(scale) & 3u) ||
      !aligned16(out))
    return MOE_EALIGN;
  if (rows > (int64_t(1) << 40) / cols || moe::int8_dequant_blocks(rows, cols) > int64_t(UINT_MAX))
    return MOE_ESHAPE;
  int st = check_device();
  if (st) return st;
  prof_begin(stream);
  return launched(moe::launch_int8_row_dequant(q, scale, rows, cols, out, stream), stream);
}

MOE_API int moe_mxfp8_quantize(const uint16_t* x, int64_t n_rows, int32_t k, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
  if (x == nullptr || codes == nullptr || scales == nullptr || n_rows <= 0 || k <= 0)
    return MOE_EINVAL;
  if (k % 32) return MOE_ESHAPE;
  if (!aligned16(x) || !aligned16(codes)) return MOE_EALIGN;
  if (uint64_t(n_rows) * uint64_t(k / 32) > (uint64_t(UINT_MAX) - 255)) return MOE_ESHAPE;
  int st = check_device();
  if (st) return st;
  prof_begin(stream);
  return launched(moe::launch_mxfp8_quantize(x, n_rows, k, codes, scales, stream), stream);
}

MOE_API int moe_set_wait_limit(int64_t polls) {
  g_wait_limit = polls < 0 ? moe::kDefaultSpinLimit : long(polls);
  return MOE_OK;
}

MOE_API int moe_workspace_status(const void* workspace, uint64_t workspace_bytes,
                                 hipStream_t stream) {
  if (workspace == nullptr || workspace_bytes < 8) return MOE_EINVAL;
  if (!aligned16(workspace)) return MOE_EALIGN;
  int st = check_device();
  if (st) return st;
  // the word is the first 8 bytes of every workspace (see carve)
  unsigned long long word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, 8, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if ((st = launched(e, stream))) return st;
  if (word != moe::kWaitGaveUp) return MOE_OK;
  const unsigned long long zero = 0;
  e = hipMemcpyAsync(const_cast<void*>(workspace), &zero, 8, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if ((st = launched(e, stream))) return st;
  return MOE_ETIMEOUT;
}

MOE_API int moe_workspace_region(const moe_layer_desc* layer, int64_t n_tokens, int32_t region,
                                 uint64_t* offset, uint64_t* bytes) {
  if (offset == nullptr || bytes == nullptr) return MOE_EINVAL;
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_tokens(n_tokens))) return st;
  const Carve c = carve(layer, n_tokens);
  const uint64_t t = uint64_t(n_tokens), k = uint64_t(layer->top_k);
  const uint64_t Kq = pad512(layer->hidden), Iq = pad512(layer->inter);
  switch (region) {
    case MOE_WS_PAIRS: *offset = c.pairs; *bytes = t * k * 4; break;
    case MOE_WS_X_CODES: *offset = c.xq; *bytes = t * Kq; break;
    case MOE_WS_X_SCALES: *offset = c.xs; *bytes = t * Kq / 32; break;
    case MOE_WS_H_CODES: *offset = c.hq; *bytes = t * k * Iq; break;
    case MOE_WS_H_SCALES: *offset = c.hs8; *bytes = t * k * Iq / 32; break;
    default: return MOE_EINVAL;
  }
  return MOE_OK;
}

MOE_API int moe_mfma_rate(int32_t a_fmt, int32_t b_fmt, int64_t iters, int32_t n_blocks,
                          float* out, hipStream_t stream) {
  if (out == nullptr || iters <= 0 || n_blocks <= 0) return MOE_EINVAL;
  if (!((a_fmt == 4 && (b_fmt == 4 || b_fmt == 0)) || (a_fmt == 0 && b_fmt == 0)))
    return MOE_EUNSUPPORTED;
  if (iters > (int64_t(1) << 40) || n_blocks > (1 << 20)) return MOE_ESHAPE;
  if (reinterpret_cast<uintptr_t>(out) & 3u) return MOE_EALIGN;
  int st = check_device();
  if (st) return st;
  prof_begin(stream);
  return launched(moe::launch_mfma_rate(a_fmt, b_fmt, iters, n_blocks, out, stream), stream);
}
