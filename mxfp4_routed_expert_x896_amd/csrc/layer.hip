// The layer's kernels.  Every launch is one role-dispatch kernel whose
// workgroups take different roles by block index, so that independent work
// shares a launch.  moe_layer on the GEMV path runs, for more than 8 tokens,
//   1. router logits            + shared experts' gate/up
//   2. top-k and plan           + shared experts' down
//   3. routed gate/up
//   4. routed down and the weighted combine;
// for 2 to 8 tokens the top-k and plan end launch 1 (on one workgroup that
// waits for the logits) and the shared down joins launch 3; one token runs
// the whole layer in one launch whose roles wait on flags (moe_decode_front).
// moe_forward (routing given) runs plan + shared gate/up, routed gate/up
// + shared down, routed down + combine.  The shared experts do not depend on
// the routing, so their weights stream while the router and the top-k run.
//
// Expert products.  Deltafin README ("An experiment in running Kimi K3 ..."),
// "Techniques / Compute": the MXFP4 weights are decoded inside the product
// instead of being dequantised to a temporary first; the Deltafin explainer
// (bhfrc.com), section 6.2, gives the reason (a separate pass costs memory
// and another trip through memory bandwidth).  Here a weight never exists in
// dequantised form outside registers.  Each lane loads 16 bytes of codes --
// one whole 32-element block of one row, so one E8M0 exponent -- converts
// them with v_cvt_scalef32_pk_bf16_fp4 (the block exponent applied in the
// convert; exact, since an E2M1 value times a power of two is a bf16,
// subnormals included) and feeds them as the A operand of
// v_mfma_f32_16x16x32_bf16.  The tokens routed to the expert are the B
// columns (up to 16 per pass), accumulation is fp32.  At batch 1 only one B
// column is live: the matrix core takes the multiply-accumulate off the
// vector ALU (one convert per code byte remains), which is what lets the
// weight stream run near the HBM roof; batched decode then reuses every
// converted weight for all tokens of the expert at no extra cost.
//
// Operand mapping (wave64, lane l: g = l / 16, c = l % 16): weights are read
// in the MFMA-tiled layout written by pack.hip, so for tile kb a wave loads
// 1 KiB of contiguous codes in which lane l holds block bi = 4 kb + g of row
// 16 rg + c; the lane's scales of four consecutive tiles are one dword of
// the scale region.  MFMA step s (0..3) takes elements 8 s .. 8 s + 7 of
// that block, i.e. contraction index K = 32 bi + 8 s + j; the B lane (g, c)
// supplies the same K indices of token c.  The 16 x 16 fp32 result leaves
// rows 4 g + i (i = 0..3) of token c in lane (g, c).  bf16 (shared)
// matrices use 1 KiB tiles of 16 rows x 32 columns, lane l holding columns
// 8 g .. 8 g + 7.
#include "common.hpp"
#include "kernels.hpp"
#include "bfgemm.hpp"
#include "mxgemm.hpp"
#include "plan.hpp"
#include "router.hpp"

namespace moe {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsD = kDownRows;  // routed down rows per workgroup (a multiple of 16)
constexpr int kRowsSD = 64;        // shared down rows per workgroup (one row group per wave)
constexpr int kCols = 16;         // B columns of one MFMA: at most 16 tokens per pass
static_assert(kCols == kGemvPassTokens, "the launcher sizes the shared roles' passes");
constexpr int kLdsBudget = 32768;  // bytes of staged activations per workgroup
// Routed gate/up: its token rows are H bf16 each (14 KiB at K3); three
// workgroups per CU (its register limit) leave 53 KiB of LDS each, three K3
// tokens, so an expert with up to three tokens streams its weights once.
constexpr int kLdsBudgetGU = 53248;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// 16 bytes stored by another workgroup of the same launch: two device-scope
// 8-byte loads (past this XCD's L2, see store_coherent).
__device__ __forceinline__ u32x4 ld16_coherent(const void* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = load_coherent(q), b = load_coherent(q + 1);
  return u32x4{uint32_t(a), uint32_t(a >> 32), uint32_t(b), uint32_t(b >> 32)};
}
template <bool kReuse>
__device__ __forceinline__ u32x4 ld_w(const void* p) {
  if constexpr (kReuse) return ld16(p);
  else return ld_nt(p);
}

__device__ __forceinline__ f32x4_t mfma(const u32x4& a, const u32x4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32 -> bf16 hi + bf16 lo with hi + lo = v to about 2^-17 relative.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(v);
  lo = f32_to_bf16(v - bf16_to_f32(hi));
}

// Counts this workgroup's arrival on *cnt once all its global stores have
// completed; true in every thread of the last of n arrivals.  With the
// stores made through the coherent level (store_coherent), the last
// workgroup then sees every other workgroup's results.
__device__ __forceinline__ bool arrive_last(int* cnt, int n) {
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == n - 1;
  }
  __syncthreads();
  return last != 0;
}

// Contraction length padded to whole 4-tile super-steps (512 columns of
// MXFP4 tiles, four 128-column groups of bf16 tiles).  Activations are
// staged zero-filled up to it, so the clamped tail loads (see load_gu)
// multiply zeros.
__host__ __device__ __forceinline__ int pad_k(int K) { return (K + 511) / 512 * 512; }

// Stage the bf16 rows of mt tokens into LDS rows of `stride` elements:
// dst[j][0..K) = src(j)[0..K), dst[j][K..Kp) = 0; sources via src(j).
template <typename Src>
__device__ __forceinline__ void stage_rows(uint16_t* dst, int stride, int mt, int K, int Kp,
                                           Src src) {
  const int nch = Kp / 8;
  for (int i = threadIdx.x; i < mt * nch; i += kThreads) {
    const int j = i / nch, q = i % nch;
    *reinterpret_cast<u32x4*>(dst + j * stride + q * 8) =
        q * 8 < K ? ld16(src(j) + q * 8) : u32x4{0, 0, 0, 0};
  }
}

// Stage packed h rows (uint32: bf16 hi in the low half, lo in the high
// half) of mt tokens into LDS as interleaved bf16 rows: row 2 j = hi and row
// 2 j + 1 = lo of token j (zero-filled from K to Kp).  As B columns of one
// MFMA, hi and lo of a token are then multiplied by the same weights in one
// instruction; hi_sum() adds the two columns afterwards.
// kCoherent: the rows were stored by other workgroups of the same launch.
template <bool kCoherent = false, typename Src>
__device__ __forceinline__ void stage_h(uint16_t* dst, int stride, int mt, int K, int Kp,
                                        Src src) {
  const int nch = Kp / 4;
  for (int i = threadIdx.x; i < mt * nch; i += kThreads) {
    const int j = i / nch, q = i % nch;
    u32x4 v = {0, 0, 0, 0};
    if (q * 4 < K) v = kCoherent ? ld16_coherent(src(j) + q * 4) : ld16(src(j) + q * 4);
    const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
    *reinterpret_cast<u32x2*>(dst + (2 * j) * stride + q * 4) =
        u32x2{(w0 & 0xFFFFu) | (w1 << 16), (w2 & 0xFFFFu) | (w3 << 16)};
    *reinterpret_cast<u32x2*>(dst + (2 * j + 1) * stride + q * 4) =
        u32x2{(w0 >> 16) | (w1 & 0xFFFF0000u), (w2 >> 16) | (w3 & 0xFFFF0000u)};
  }
}

// Sum of the MFMA result columns c and c ^ 1 (a token's hi and lo parts),
// valid in the even lane of each pair.
__device__ __forceinline__ float hi_lo_sum(float v) {
  return v + __uint_as_float(dpp_or_zero<0xB1, 0xF>(__float_as_uint(v)));  // quad_perm [1,0,3,2]
}

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Wave index within the workgroup as a scalar (uniform) value, so that loop
// bounds and tile addresses derived from it stay in scalar registers.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
}

// Two-stage software pipeline over steps s0 .. s1 - 1 with two register
// buffers used alternately: while step s is computed from one buffer, the
// loads of step s + 1 are in flight into the other.  The caller has issued
// load(a, s0).  Two things keep the loads of step s + 1 in flight while
// step s computes: the buffers alternate instead of being copied (a copy
// would wait for them), and the steady-state loop issues its loads without
// conditions, so the compiler can count exactly how many are outstanding
// (loads under a branch make it wait for all of them).
template <typename Buf, typename Load, typename Comp>
__device__ __forceinline__ void pipeline2(int s0, int s1, Buf& a, Buf& b, Load load, Comp comp) {
  int s = s0;
  for (; s + 2 < s1; s += 2) {
    load(b, s + 1);
    __builtin_amdgcn_sched_barrier(0);  // loads stay ahead of the wait (see pipelineN)
    comp(a, s);
    load(a, s + 2);
    __builtin_amdgcn_sched_barrier(0);
    comp(b, s + 1);
  }
  if (s + 1 < s1) {
    load(b, s + 1);
    comp(a, s);
    comp(b, s + 1);
  } else if (s < s1) {
    comp(a, s);
  }
}

// D-stage version: a ring of D register buffers, loads issued D - 1 steps
// ahead of the step being computed.  The caller has issued nothing; the
// prologue loads the first D - 1 steps.  Steady-state loads are
// unconditional for the same reason as in pipeline2.  mid() runs after the
// prologue's loads are issued (for work that overlaps them, e.g. staging).
template <int D, typename Buf, typename Load, typename Mid, typename Comp>
__device__ __forceinline__ void pipelineN(int s0, int s1, Buf (&b)[D], Load load, Mid mid,
                                          Comp comp) {
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (s0 + d < s1) load(b[d], s0 + d);
  mid();
  int s = s0;
  for (; s + 2 * D - 1 <= s1; s += D) {  // all D prefetches of this round exist
#pragma unroll
    for (int d = 0; d < D; ++d) {
      load(b[(d + D - 1) % D], s + d + D - 1);
      // keep the loads ahead of the wait for step s + d: scheduled after
      // it, they would leave one step fewer in flight
      __builtin_amdgcn_sched_barrier(0);
      comp(b[d], s + d);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {  // remaining < 2 D - 1 steps, conditions allowed
    if (s + d >= s1) break;
    if (s + d + D - 1 < s1) load(b[(d + D - 1) % D], s + d + D - 1);
    comp(b[d], s + d);
  }
  s += D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (s + d >= s1) break;
    comp(b[d], s + d);
  }
}

// ------------------------------------------------------------------------
// Waits until flags[0 .. n) and flags2[0 .. n2) all hold this call's epoch
// (both polled in one round trip), or gives up after L.spin_limit polls and
// sets the workspace status marker (the caller reads it with
// moe_workspace_status; the work then runs on what is there: wrong results,
// no hang).  Every thread of the workgroup calls it.
__device__ void wait_flags(const GemvLayer& L, const unsigned long long* flags, int n,
                           const unsigned long long* flags2 = nullptr, int n2 = 0) {
  bool done = false;
  for (long it = 0; it < L.spin_limit && !done; ++it) {
    int ok = 1;
    for (int i = threadIdx.x; i < n + n2; i += kThreads)
      ok &= load_coherent(i < n ? &flags[i] : &flags2[i - n]) == L.epoch;
    done = __syncthreads_and(ok) != 0;
    if (!done) __builtin_amdgcn_s_sleep(8);
  }
  if (threadIdx.x == 0 && !done) store_coherent(L.status, kWaitGaveUp);
}

// ------------------------------------------------------------------------
// Gate/up.  Workgroup = (expert, 32 rows): wave w takes row group w / 2 of
// the tile and half w % 2 of the contraction; the halves meet in LDS.  The
// tokens' x rows are staged in LDS (B operand), mtp at a time.  Weight
// tiles are double-buffered (pipeline2): the loads of super-step kq + 1 are
// in flight while super-step kq is converted and multiplied.

struct GuTiles {
  u32x4 g[4], u[4];
  uint32_t sg, su;
};

// Tiles past the row group's last (kb >= nkb, only when nkb is not a
// multiple of 4) are loaded from the last tile instead: a valid address and
// no branch; their scale bytes are the 127 padding and the staged
// activations there are zero, so they add nothing.
__device__ __forceinline__ void load_gu(GuTiles& t, const uint8_t* gcodes, const uint8_t* ucodes,
                                        const uint8_t* gscl, const uint8_t* uscl, int kq, int nkb,
                                        int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kb = min(4 * kq + j, nkb - 1);
    t.g[j] = ld_nt(gcodes + size_t(kb) * 1024 + 16 * lane);
    t.u[j] = ld_nt(ucodes + size_t(kb) * 1024 + 16 * lane);
  }
  t.sg = *reinterpret_cast<const uint32_t*>(gscl + 256 * kq);
  t.su = *reinterpret_cast<const uint32_t*>(uscl + 256 * kq);
}

__device__ __forceinline__ void mma_gu(const GuTiles& t, const uint16_t* xrow, int kq, int g,
                                       f32x4_t& ag, f32x4_t& au) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bi = 16 * kq + 4 * j + g;
    const float sg = e8m0_to_f32((t.sg >> (8 * j)) & 0xFFu);
    const float su = e8m0_to_f32((t.su >> (8 * j)) & 0xFFu);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 bx = lds16(xrow + bi * 32 + 8 * s);
      ag = mfma(fp4x8_scaled(t.g[j][s], sg), bx, ag);
      au = mfma(fp4x8_scaled(t.u[j][s], su), bx, au);
    }
  }
}

// Adds the tiles of waves 1..3 into wave 0 (contraction split in four).
__device__ __forceinline__ void join_quarters(f32x4_t& a, f32x4_t& b, float* red) {
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  __syncthreads();
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[(wave * kWave + lane) * 8 + i] = a[i];
      red[(wave * kWave + lane) * 8 + 4 + i] = b[i];
    }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] += red[(w * kWave + lane) * 8 + i];
        b[i] += red[(w * kWave + lane) * 8 + 4 + i];
      }
    }
  }
}

// Adds the partner half's tiles (wave w ^ 1) into waves with even index.
__device__ __forceinline__ void join_halves(f32x4_t& a, f32x4_t& b, float* red) {
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  __syncthreads();
  if (wave & 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[(wave * kWave + lane) * 8 + i] = a[i];
      red[(wave * kWave + lane) * 8 + 4 + i] = b[i];
    }
  }
  __syncthreads();
  if (!(wave & 1)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] += red[((wave + 1) * kWave + lane) * 8 + i];
      b[i] += red[((wave + 1) * kWave + lane) * 8 + 4 + i];
    }
  }
}

// One-token front: the expert of slot a, once the top-k of this launch has
// stored its tagged word (bounded like wait_flags; a give-up sets the status
// marker and returns what is there, clamped by the caller).  Every thread of
// the workgroup calls it.
__device__ int front_expert(const GemvLayer& L, int a) {
  const unsigned long long tag = L.epoch & 0xFFFFFFFFFFFFull;
  unsigned long long v = 0;
  bool done = false;
  for (long it = 0; it < L.spin_limit && !done; ++it) {
    v = load_coherent(&L.idtag[a]);
    done = __syncthreads_and((v >> 16) == tag) != 0;
    if (!done) __builtin_amdgcn_s_sleep(8);
  }
  if (threadIdx.x == 0 && !done) store_coherent(L.status, kWaitGaveUp);
  return __builtin_amdgcn_readfirstlane(int(v & 0xFFFFu));
}

// Expert slot a of the routed launches: the number of live slots, its
// expert and its plan positions [p0, p1).  The plan reads are issued
// together (all in bounds for any a < E) and the slot is checked after they
// land, so the expert's first weight loads wait for one round trip.
__device__ __forceinline__ void slot_of(const GemvLayer& L, int a, int& n, int& e, int& p0,
                                        int& p1) {
  if (L.direct) {
    n = L.T * L.k;
    // in the front launch the top-k of this launch stores it (tagged word)
    const int id = L.front ? front_expert(L, min(a, n - 1)) : L.ids_in[min(a, n - 1)];
    e = min(max(id, 0), L.E - 1);  // clamped like the plan's ids
    p0 = a;
    p1 = a + 1;
    return;
  }
  n = L.plan.n_active[0];
  e = L.plan.active[a];
  p0 = L.plan.act_off[a];
  p1 = L.plan.act_off[a + 1];
}

// Pair (token * k + slot) at plan position p.
__device__ __forceinline__ int pair_at(const GemvLayer& L, int p) {
  return L.direct ? p : L.plan.pairs[p];
}

// Packed record of expert e: record e, or with an expert pool the record
// its slot map names (clamped to the pool).
__device__ __forceinline__ const uint8_t* record_of(const GemvLayer& L, int e) {
  const int r = L.eslot != nullptr ? min(max(L.eslot[e], 0), L.n_slots - 1) : e;
  return L.experts + size_t(r) * L.stride;
}

// kFront: in the one-token front launch; the h rows are stored through the
// coherent level and flagged for the routed down of the same launch
// (guflags[a * I/32 + tile]).
template <bool kFront = false>
__device__ void routed_gateup(const GemvLayer& L, int a, int tile, uint16_t* xs, float* red) {
  int na, e, p0, p1;
  slot_of(L, a, na, e, p0, p1);
  if (a >= na) return;
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, I = L.I;
  const PackedMx pm(I, H);
  const int nkq = pm.nkb4 / 4;
  const int kqh = (nkq + 1) / 2;
  const int kq0 = (wave & 1) * kqh, kq1 = min(kq0 + kqh, nkq);
  const int rg = tile * 2 + wave / 2;
  const uint8_t* gbase = record_of(L, e);
  const uint8_t* ubase = gbase + pm.bytes;
  const uint8_t* gcodes = gbase + size_t(rg) * pm.nkb * 1024;
  const uint8_t* ucodes = ubase + size_t(rg) * pm.nkb * 1024;
  const uint8_t* gscl = gbase + pm.scale_dword(rg, 0, lane);
  const uint8_t* uscl = ubase + pm.scale_dword(rg, 0, lane);
  const int xstride = pad_k(H) + 8;

  for (int t0 = p0; t0 < p1; t0 += L.mtp_gu) {
    const int mt = min(L.mtp_gu, p1 - t0);
    GuTiles ta, tb;
    auto load = [&](GuTiles& t, int kq) { load_gu(t, gcodes, ucodes, gscl, uscl, kq, pm.nkb, lane); };
    if (kq0 < kq1) load(ta, kq0);
    __syncthreads();
    stage_rows(xs, xstride, mt, H, pad_k(H), [&](int j) {
      return L.x + size_t(min(pair_at(L, t0 + j) / L.k, L.T - 1)) * H;
    });
    __syncthreads();
    const uint16_t* xrow = xs + (c < mt ? c : 0) * xstride;
    f32x4_t ag = {0.0f, 0.0f, 0.0f, 0.0f}, au = {0.0f, 0.0f, 0.0f, 0.0f};
    pipeline2(kq0, kq1, ta, tb, load,
              [&](const GuTiles& t, int kq) { mma_gu(t, xrow, kq, g, ag, au); });
    join_halves(ag, au, red);
    if (!(wave & 1) && c < mt) {
      uint32_t hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t hi, lo;
        split_bf16(silu(ag[i]) * au[i], hi, lo);
        hv[i] = uint32_t(hi) | (uint32_t(lo) << 16);
      }
      uint32_t* hrow = L.h + size_t(t0 + c) * I + rg * 16 + 4 * g;
      if (kFront) {  // read by the routed down of this launch
        store_coherent(reinterpret_cast<uint64_t*>(hrow), uint64_t(hv[0]) | uint64_t(hv[1]) << 32);
        store_coherent(reinterpret_cast<uint64_t*>(hrow) + 1,
                       uint64_t(hv[2]) | uint64_t(hv[3]) << 32);
      } else {
        *reinterpret_cast<u32x4*>(hrow) = u32x4{hv[0], hv[1], hv[2], hv[3]};
      }
    }
  }
  if (kFront) {  // h rows stored: flag them for the routed down of slot a
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) store_coherent(&L.guflags[a * (I / 32) + tile], L.epoch);
  }
}

// Shared down waves keep this many super-steps of weights in flight; the
// shared down shares its launch with the routed gate/up, whose occupancy
// (three waves per SIMD) its registers must not lower.
constexpr int kSharedDownStages = 3;

// Shared gate/up (bf16): 1 KiB tiles of 16 rows x 32 columns are the A
// operand as loaded; four tiles per super-step, three in flight.  A bf16
// row is 3.8x the bytes of an MXFP4 row, so a workgroup takes one row group
// and its four waves split the contraction in quarters (more waves in
// flight for the same bytes).  The B operand (16 tokens per pass) is read
// straight from the token rows, which every workgroup shares through L2:
// per tile it is as many bytes as the weights, so no LDS staging (and no
// cap on tokens per pass from the LDS size) is needed.
// kReuse: more than one pass of tokens, so the weights are loaded with the
// default cache policy and later passes find them in the caches; a single
// pass streams them past the caches.  D: super-steps in flight.
// Tokens p0 .. p1 - 1 (p1 < 0: all), kCols per pass.
template <bool kReuse, int D = 3>
__device__ void shared_gateup(const GemvLayer& L, int sx, int rg, float* red, int p0 = 0,
                              int p1 = -1) {
  if (p1 < 0) p1 = L.T;
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, I = L.I;
  const int nu = H / 32;
  const int nq = (nu + 3) / 4;
  const int qq = (nq + kWaves - 1) / kWaves;
  const int q0 = min(wave * qq, nq), q1 = min(q0 + qq, nq);
  const uint16_t* gt = L.sgate + sx * (size_t(I) * H) + size_t(rg) * nu * 512;
  const uint16_t* ut = L.sup + sx * (size_t(I) * H) + size_t(rg) * nu * 512;
  const size_t plane = size_t(L.S) * L.T * I;
  struct Tiles {
    u32x4 g[4], u[4], x[4];
  };
  for (int t0 = p0; t0 < p1; t0 += kCols) {
    const int mt = min(kCols, p1 - t0);
    // B straight from the token rows (L2-resident): lane (c, g) reads token
    // c's 8 columns of each 32-column tile (a clamped token past mt)
    const uint16_t* xrow = L.x + size_t(t0 + min(c, mt - 1)) * H + 8 * g;
    auto load = [&](Tiles& t, int q) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int u = min(4 * q + j, nu - 1);  // past the end: skipped below
        t.g[j] = ld_w<kReuse>(gt + size_t(u) * 512 + 8 * lane);
        t.u[j] = ld_w<kReuse>(ut + size_t(u) * 512 + 8 * lane);
        t.x[j] = ld16(xrow + u * 32);
      }
    };
    Tiles bufs[D];
    f32x4_t ag = {0.0f, 0.0f, 0.0f, 0.0f}, au = {0.0f, 0.0f, 0.0f, 0.0f};
    pipelineN<D>(q0, q1, bufs, load, [&]() {}, [&](const Tiles& t, int q) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (4 * q + j >= nu) break;  // uniform
        ag = mfma(t.g[j], t.x[j], ag);
        au = mfma(t.u[j], t.x[j], au);
      }
    });
    join_quarters(ag, au, red);
    if (wave == 0 && c < mt) {
      uint64_t hi4 = 0, lo4 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t hi, lo;
        split_bf16(silu(ag[i]) * au[i], hi, lo);
        hi4 |= uint64_t(hi) << (16 * i);
        lo4 |= uint64_t(lo) << (16 * i);
      }
      // rows 4 g .. 4 g + 3: one 8-byte store per part (through the coherent
      // level: in the front launch the shared down reads them)
      const size_t o = (size_t(sx) * L.T + t0 + c) * I + rg * 16 + 4 * g;
      store_coherent(reinterpret_cast<uint64_t*>(L.hs + o), hi4);
      store_coherent(reinterpret_cast<uint64_t*>(L.hs + plane + o), lo4);
    }
  }
  if (L.front) {  // h rows stored: flag them for the shared down of this launch
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) store_coherent(&L.sgflags[sx * (I / 16) + rg], L.epoch);
  }
}

// Router logits of kRouterSplitMin or more tokens: bf16 MFMA with 16 experts'
// router rows as A, straight from their row-major storage (lane (c, g) reads
// row c at columns 32 u + 8 g .. + 7, the packed-tile layout), and 16 tokens
// of x as B from L2.  Workgroup b takes experts 16 (b / kRouterSplit) .. + 15
// and quarter q = b % kRouterSplit of the contraction; wave w takes slice
// 4 q + w of 16 slices of the 32-column tiles and keeps its slice of the rows
// in registers for every token group.  The waves' sums are added in wave
// order and the quarter's partial logits stored (quarter 0 adds the bias);
// the top-k adds the quarters in order.  The token rows, not the router
// rows, are what repeats per token group, and they are L2-resident.
constexpr int kRsTiles = 16;  // tiles per slice: H <= 8192 = 16 slices x 16 tiles x 32
__device__ void router_split_role(const GemvLayer& L, int b, float* red) {
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, E = L.E, T = L.T;
  const int e0 = (b / kRouterSplit) * 16, q = b % kRouterSplit;
  const int nt = H / 32;
  const int sl = q * kWaves + wave;
  const int t_beg = sl * nt / 16, n_i = (sl + 1) * nt / 16 - t_beg;  // uniform, <= kRsTiles
  const uint16_t* arow = L.wr + size_t(min(e0 + c, E - 1)) * H + 8 * g;
  u32x4 a[kRsTiles];
#pragma unroll
  for (int i = 0; i < kRsTiles; ++i) a[i] = ld_nt(arow + 32 * min(t_beg + i, nt - 1));
  float* part = L.logits + size_t(q) * T * E;
  for (int t0 = 0; t0 < T; t0 += 16) {
    const uint16_t* xrow = L.x + size_t(min(t0 + c, T - 1)) * H + 8 * g;
    u32x4 bx[kRsTiles];
#pragma unroll
    for (int i = 0; i < kRsTiles; ++i) bx[i] = ld16(xrow + 32 * min(t_beg + i, nt - 1));
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kRsTiles; ++i)
      if (i < n_i) acc = mfma(a[i], bx[i], acc);  // uniform
    __syncthreads();  // red is free
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * kWave + lane) * 4 + r] = acc[r];
    __syncthreads();
    if (wave == 0 && t0 + c < T) {
      // lane (c, g) holds experts e0 + 4 g .. + 3 of token t0 + c
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + 4 * g + r;
        float v = red[lane * 4 + r];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) v += red[(ww * kWave + lane) * 4 + r];
        if (q == 0 && L.rbias != nullptr && e < E) v += L.rbias[e];
        // through the coherent level: the top-k of up to kSelwMaxTokens
        // tokens reads it in the same launch
        if (e < E) store_coherent(&part[size_t(t0 + c) * E + e], v);
      }
    }
  }
}

// ------------------------------------------------------------------------
// Down projections and the combine.  Workgroups are (expert, tile of kRowsD
// output rows, 16 per wave); h enters as bf16 hi + lo, staged in LDS (the
// shared down reads it straight from L2, 8 tokens per pass, hi and lo as
// adjacent B columns).  The shared experts' down runs in an earlier launch and
// leaves fp32 outputs in ysh.  Each routed workgroup writes fp32 partials
// for its rows and tokens; the last one to finish a tile (device-scope
// counter, zeroed by the plan builder of the same call) sums the tile's
// partials in a fixed order -- routed slots j = 0..k-1 weighted by w, then
// the shared experts, then the residual -- and writes the bf16 output.  The
// sum order does not depend on which workgroup arrives last, so the output
// is deterministic.

struct DnTiles {
  u32x4 w[4];
  uint32_t sc;
};

// Routed down: three stages (8 KiB per wave in flight) keep the kernel
// under 128 VGPRs, so four waves share a SIMD; at the K3 shape (I = 1536)
// a wave streams 2 row groups x 3 super-steps of 4 KiB, and more waves in
// flight per SIMD beat deeper pipelines per wave (measured).
constexpr int kDownStages = 3;
// In the one-token front launch (two waves per SIMD, the front's register
// budget) a wave keeps six steps in flight, the first five issued before the
// wait for the slot's h.
constexpr int kDownStagesFront = 6;
// Shared gate/up super-steps in flight in the front launch.
constexpr int kSharedStagesFront = 3;
// Waves per SIMD the front launch's registers are fitted to.
constexpr int kFrontWaves = 2;

// Routed down: workgroup = (expert, tile of kRowsD rows); wave w takes the
// tile's row groups w, w + 4, w + 8, ... one after the other as one continuous
// pipeline of (row group, super-step) steps, so its loads never drain
// between row groups; a row group's partials are stored after its last
// super-step.  kFront: in the front launch, h is waited for (the slot's
// gate/up flags) and read through the coherent level once the prologue's
// weight loads are in flight.
template <int D, bool kFront>
__device__ void routed_down(const GemvLayer& L, int a, int e, int p0, int p1, int tile,
                            uint16_t* hsm) {
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, I = L.I;
  const PackedMx pgu(I, H), pd(H, I);
  const int nkq = pd.nkb4 / 4;
  // the tile's row groups rg0 + wave + kWaves r, r = 0 .. nrg - 1
  constexpr int R = kFront ? kFrontDownRows : kRowsD;  // rows per tile
  const int tile_rg = min(R / 16, H / 16 - tile * (R / 16));  // ragged last tile
  const int rg0 = tile * (R / 16) + wave;
  const int nrg = max(0, (tile_rg - wave + kWaves - 1) / kWaves);
  const int nsteps = nrg * nkq;
  const uint8_t* base = record_of(L, e) + 2 * pgu.bytes;
  const uint8_t* codes = base + size_t(rg0) * pd.nkb * 1024 + 16 * lane;
  const uint8_t* scl = base + pd.scale_dword(rg0, 0, lane);
  const int hstride = pad_k(I) + 8;
  auto load = [&](DnTiles& t, int s) {
    const int r = s / nkq, kq = s - r * nkq;
    const uint8_t* cr = codes + size_t(r) * kWaves * pd.nkb * 1024;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t.w[j] = ld_nt(cr + size_t(min(4 * kq + j, pd.nkb - 1)) * 1024);
    t.sc = *reinterpret_cast<const uint32_t*>(scl + size_t(r) * kWaves * pd.nsup * 256 + 256 * kq);
  };

  for (int t0 = p0; t0 < p1; t0 += L.mtp_d) {
    const int mt = min(L.mtp_d, p1 - t0);
    DnTiles bufs[D];
    const uint16_t* bh = hsm + (c < 2 * mt ? c : 0) * hstride;  // column c: token c / 2, hi / lo
    const int tok = c / 2;
    const int pair = pair_at(L, t0 + (tok < mt ? tok : 0));
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto stage = [&]() {
      __syncthreads();
      if constexpr (kFront) wait_flags(L, L.guflags + a * (I / 32), I / 32);
      stage_h<kFront>(hsm, hstride, mt, I, pad_k(I),
                      [&](int j) { return L.h + size_t(t0 + j) * I; });
      __syncthreads();
    };
    pipelineN<D>(0, nsteps, bufs, load, stage, [&](const DnTiles& t, int s) {
      const int r = s / nkq, kq = s - r * nkq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bi = 16 * kq + 4 * j + g;
        const float sd = e8m0_to_f32((t.sc >> (8 * j)) & 0xFFu);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc = mfma(fp4x8_scaled(t.w[j][q], sd), lds16(bh + bi * 32 + 8 * q), acc);
      }
      if (kq == nkq - 1) {  // row group rg0 + kWaves r complete
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = hi_lo_sum(acc[i]);
        if ((c & 1) == 0 && tok < mt) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            store_coherent(&L.part[size_t(pair) * H + (rg0 + kWaves * r) * 16 + 4 * g + i], y[i]);
        }
        acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    });
  }
}

// Arrivals that complete front tile ft (kFrontDownRows rows) of one token:
// the k routed down workgroups and the shared down workgroups of its rows.
__device__ __forceinline__ int front_arrivals(const GemvLayer& L, int ft) {
  constexpr int per = kFrontDownRows / kRowsSD;
  return L.T * L.k + L.S * min(per, L.n_stiles - per * ft);
}
template <int R, bool kFront>
__device__ void combine_tile(const GemvLayer& L, int tile);

template <bool kReuse>  // as for shared_gateup; tokens p0 .. p1 - 1, kCols / 2 per pass
__device__ void shared_down(const GemvLayer& L, int sx, int tile, int p0 = 0, int p1 = -1) {
  if (p1 < 0) p1 = L.T;
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int rg = tile * (kRowsSD / 16) + wave;
  const bool live = rg < L.H / 16;
  const int H = L.H, I = L.I;
  const int nu = I / 32;
  const int nq = (nu + 3) / 4;
  const uint16_t* dt = L.sdown + sx * (size_t(H) * I) + size_t(live ? rg : 0) * nu * 512;
  const size_t plane = size_t(L.S) * L.T * I;
  struct Tiles {
    u32x4 w[4], h[4];
  };
  for (int t0 = p0; t0 < p1; t0 += kCols / 2) {
    const int mt = min(kCols / 2, p1 - t0);
    // B straight from h (L2-resident): column c is token c / 2's hi (c even)
    // or lo (c odd) part; lane (c, g) reads 8 columns of each 32-column tile
    const int tok = t0 + min(c / 2, mt - 1);
    const uint16_t* hrow = L.hs + (c & 1) * plane + (size_t(sx) * L.T + tok) * I + 8 * g;
    auto load = [&](Tiles& t, int q) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int u = min(4 * q + j, nu - 1);  // past the end: skipped below
        t.w[j] = ld_w<kReuse>(dt + size_t(u) * 512 + 8 * lane);
        t.h[j] = ld16(hrow + u * 32);
      }
    };
    Tiles bufs[kSharedDownStages];
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    pipelineN<kSharedDownStages>(0, live ? nq : 0, bufs, load, [&]() {}, [&](const Tiles& t, int q) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (4 * q + j >= nu) break;  // uniform
        acc = mfma(t.w[j], t.h[j], acc);
      }
    });
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = hi_lo_sum(acc[i]);
    if (live && (c & 1) == 0 && c / 2 < mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        L.ysh[(size_t(sx) * L.T + t0 + c / 2) * H + rg * 16 + 4 * g + i] = y[i];
    }
  }
}

// Shared down in the one-token front launch: workgroup = (shared expert sx,
// 64 rows), wave w takes row group 4 tile + w.  The weight loads of the
// pipeline's first steps are issued before the wait for the shared
// expert's gate/up flags (and the top-k's, which clears the arrival
// counters), both polled in one round trip; the token's h (hi and lo rows)
// is then staged in LDS from the coherent level.  The rows are stored
// through the coherent level and counted on their front tile, whose last
// arriver combines it.
__device__ void shared_down_front(const GemvLayer& L, int sx, int tile, uint16_t* hsm) {
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int rg = tile * (kRowsSD / 16) + wave;
  const bool live = rg < L.H / 16;
  const int H = L.H, I = L.I;
  const int nu = I / 32;
  const int nq = (nu + 3) / 4;
  const int hp = pad_k(I);  // staged row length (zeros past I)
  const uint16_t* dt = L.sdown + sx * (size_t(H) * I) + size_t(live ? rg : 0) * nu * 512;
  const size_t plane = size_t(L.S) * L.T * I;
  struct Tiles {
    u32x4 w[4];
  };
  auto load = [&](Tiles& t, int q) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t.w[j] = ld_nt(dt + size_t(min(4 * q + j, nu - 1)) * 512 + 8 * lane);
  };
  auto stage = [&]() {
    wait_flags(L, L.sgflags + sx * (I / 16), I / 16, L.idsflag, 1);
    for (int i = threadIdx.x; i < 2 * (hp / 8); i += kThreads) {
      const int r = i / (hp / 8), q = i % (hp / 8);
      u32x4 v = {0, 0, 0, 0};
      if (q * 8 < I) v = ld16_coherent(L.hs + r * plane + size_t(sx) * L.T * I + q * 8);
      *reinterpret_cast<u32x4*>(hsm + r * hp + q * 8) = v;
    }
    __syncthreads();
  };
  // B column c: the token's hi (c even) or lo (c odd) row
  const uint16_t* bh = hsm + (c & 1) * hp + 8 * g;
  Tiles bufs[kSharedDownStages];
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  pipelineN<kSharedDownStages>(0, live ? nq : 0, bufs, load, stage, [&](const Tiles& t, int q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (4 * q + j >= nu) break;  // uniform
      acc = mfma(t.w[j], lds16(bh + (4 * q + j) * 32), acc);
    }
  });
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = hi_lo_sum(acc[i]);
  if (live && c == 0) {
    float* yrow = L.ysh + size_t(sx) * L.T * H + rg * 16 + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) store_coherent(yrow + i, y[i]);
  }
  const int ft = tile / (kFrontDownRows / kRowsSD);
  if (arrive_last(&L.tile_cnt[ft], front_arrivals(L, ft)))
    combine_tile<kFrontDownRows, true>(L, ft);
}

// The last routed workgroup of a tile sums the partials into the bf16 output.
// All of a token's partial loads are issued before the first add, so the
// tail costs one memory round trip, not k of them.
// R: rows per tile; kFront: the shared outputs were stored in the same
// launch (read through the coherent level).
template <int R, bool kFront>
__device__ void combine_tile(const GemvLayer& L, int tile) {
  const int H = L.H, k = L.k;
  const int n_out = L.T * R;
  // Every load of a token's sum is issued unconditionally, with clamped
  // indices and stand-in rows for absent operands, and their values are taken
  // at one point: a load under a condition would be waited for on its own,
  // one memory round trip each.
  const float* ysh = L.S > 0 ? L.ysh : L.part;
  const uint16_t* res = L.residual != nullptr ? L.residual : L.x;
  for (int idx = threadIdx.x; idx < n_out; idx += kThreads) {
    const int t = idx / R;
    const int n = tile * R + idx % R;
    if (n >= H) continue;
    float acc = 0.0f;
    float sv[4];
    uint16_t rv = 0;
    for (int j0 = 0; j0 < k; j0 += 16) {
      float pv[16], wv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const size_t p = size_t(t) * k + min(j0 + j, k - 1);
        pv[j] = load_coherent(&L.part[p * H + n]);
        wv[j] = kFront ? load_coherent(&L.w[p]) : L.w[p];  // front: the top-k's, same launch
      }
      if (j0 == 0) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float* q = ysh + (size_t(max(min(s, L.S - 1), 0)) * L.T + t) * H + n;
          sv[s] = kFront ? load_coherent(q) : *q;
        }
        rv = res[size_t(t) * H + n];
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(pv[j]), "+v"(wv[j]));
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j0 + j < k) acc = fmaf(wv[j], pv[j], acc);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (s < L.S) acc += sv[s];
    if (L.residual != nullptr) acc += bf16_to_f32(rv);
    L.y[size_t(t) * H + n] = f32_to_bf16(acc);
  }
}


// ------------------------------------------------------------------------
// Role dispatch.  A launch's grid is the concatenation, in this order, of
// the role segments present in it (Stage counts, 0 = absent).

enum : unsigned {
  kRoleLogits = 1u,       // router logits, 4 experts per workgroup (split: 16 x a quarter)
  kRoleSelect = 2u,       // top-k, 4 tokens per workgroup (+ plan by the last)
  kRolePlan = 4u,         // plan from a given routing (one workgroup)
  kRoleSharedGU = 8u,     // shared gate/up, (expert, 16 rows) per workgroup
  kRoleSharedDown = 16u,  // shared down, (expert, 64 rows) per workgroup
  kRoleRoutedGU = 32u,    // routed gate/up, (active slot, 32 rows)
  kRoleRoutedDown = 64u,  // routed down, (active slot, kRowsD rows) + combine
  kRoleQuantX = 128u,     // prefill: x -> MXFP8 (256 blocks per workgroup)
  kRoleMxGateUp = 256u,   // prefill: routed gate/up, (token tile, 256 rows), 8 waves
  kRoleMxDown = 512u,     // prefill: routed down, (token tile, 512 rows), 8 waves
  kRoleCombine = 1024u,   // prefill: combine, one token per workgroup
  kRoleRouterMx = 2048u,  // prefill: router logits, (256 experts, 64 tokens)
  kRoleSharedGUMx = 4096u,    // prefill: shared gate/up, 2 x (expert, 128 rows, 64 tokens)
  kRoleSharedDownMx = 8192u,  // prefill: shared down, 2 x (expert, 256 rows, 64 tokens)
  kRoleSelectWait = 16384u,   // top-k of T <= 8 tokens once this launch's logits are flagged
};

// XCD-aware order for a grid over (pair, token tile): block b runs on XCD
// b % 8 (the dispatcher's round robin), so pairs are dealt out to XCDs and
// each XCD walks its pairs with the token tile fastest.  The workgroups
// sharing a weight slice then run together on one XCD and read it through
// its L2 once.  Returns false for the padding blocks.
__device__ __forceinline__ bool xcd_split(int b, int n_pairs, int n_tt, int& pair, int& tt) {
  const int xcd = b % 8, i = b / 8;
  pair = xcd + 8 * (i / n_tt);
  tt = i % n_tt;
  return pair < n_pairs;
}
__host__ __device__ __forceinline__ int xcd_grid(int n_pairs, int n_tt) {
  return 8 * ((n_pairs + 7) / 8) * n_tt;
}

// Prefill router: logits for 256 experts (4 row groups per wave, read from
// the row-major router weights) x 64 tokens, plus the bias.
__device__ void router_mx_role(const GemvLayer& L, int b, uint8_t* lds) {
  if (b == 0 && threadIdx.x == 0 && L.sel_cnt != nullptr) L.sel_cnt[0] = 0;
  const int n_tt = (L.T + bf::kTok - 1) / bf::kTok;
  const int rt = b / n_tt, tt = b % n_tt;
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, E = L.E;
  const int rg0 = rt * 16 + 4 * wave;
  const int t0 = tt * bf::kTok;
  const int nkt = H / 32;
  bf::f32x4 acc[bf::kNS][bf::kSub];
  bf::gemm_tile<1>(
      acc,
      [&](int s, int kt) {
        const int row = min((rg0 + s) * 16 + c, E - 1);
        return L.wr + size_t(row) * H + 32 * min(kt, nkt - 1) + 8 * g;
      },
      H, lds, [&](int, int j) { return L.x + size_t(min(t0 + j, L.T - 1)) * H; });
#pragma unroll
  for (int u = 0; u < bf::kSub; ++u) {
    const int t = t0 + 16 * u + c;
    if (t >= L.T) continue;
#pragma unroll
    for (int s = 0; s < bf::kNS; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (rg0 + s) * 16 + 4 * g + i;
        if (e < E) L.logits[size_t(t) * E + e] = acc[s][u][i] + (L.rbias ? L.rbias[e] : 0.0f);
      }
    }
  }
}

// The shared-expert tiles of an 8-wave workgroup of the prefill GEMM
// launches: each half (4 waves) takes one (weight slice, 64-token tile);
// block b takes token tiles 2 i, 2 i + 1 of its slice (xcd_split over
// half as many token tiles), so both halves read the same weights.  A half
// without a tile repeats the other's and stores nothing (valid = false):
// the halves share the workgroup's barriers.  lds: this half's buffers.
__device__ __forceinline__ bool shared_mx_unit(int b, int n_pairs, int n_tt, int& pair, int& tt,
                                               bool& valid) {
  const int half = threadIdx.x / (kWave * 4);
  int t2;
  if (!xcd_split(b, n_pairs, (n_tt + 1) / 2, pair, t2)) return false;
  tt = 2 * t2 + half;
  valid = tt < n_tt;
  tt = min(tt, n_tt - 1);
  return true;
}

// Prefill shared gate/up: (shared expert, 128 rows of I, 64 tokens) per
// half workgroup; wave w of the half takes row groups 2 w, 2 w + 1 of gate
// and up.  h = SiLU(g) * u leaves as bf16 hi + lo, as on the decode path.
__device__ __forceinline__ void shared_gu_mx_role(const GemvLayer& L, int b, uint8_t* lds) {
  const int n_rt = (L.I + 127) / 128, n_tt = (L.T + bf::kTok - 1) / bf::kTok;
  int pair, tt;
  bool valid;
  if (!shared_mx_unit(b, L.S * n_rt, n_tt, pair, tt, valid)) return;
  lds += (threadIdx.x / (kWave * 4)) * 2 * bf::kStageBytes;
  const int sx = pair / n_rt, rt = pair % n_rt;
  const int wave = bf::group_wave();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, I = L.I;
  const int nu = H / 32, ngroups = I / 16;
  const int rg0 = rt * 8 + 2 * wave;
  const int t0 = tt * bf::kTok;
  const uint16_t* mats[2] = {L.sgate + size_t(sx) * I * H, L.sup + size_t(sx) * I * H};
  bf::f32x4 acc[bf::kNS][bf::kSub];
  bf::gemm_tile<1>(
      acc,
      [&](int s, int kt) {
        const int rg = min(rg0 + (s & 1), ngroups - 1);
        return mats[s >> 1] + (size_t(rg) * nu + min(kt, nu - 1)) * 512 + 8 * lane;
      },
      H, lds, [&](int, int j) { return L.x + size_t(min(t0 + j, L.T - 1)) * H; });
  if (rg0 >= ngroups || !valid) return;
  const size_t plane = size_t(L.S) * L.T * I;
#pragma unroll
  for (int u = 0; u < bf::kSub; ++u) {
    const int t = t0 + 16 * u + c;
    if (t >= L.T) continue;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint32_t hi[2] = {0, 0}, lo[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t h16, l16;
        split_bf16(silu(acc[r][u][i]) * acc[2 + r][u][i], h16, l16);
        hi[i / 2] |= uint32_t(h16) << (16 * (i % 2));
        lo[i / 2] |= uint32_t(l16) << (16 * (i % 2));
      }
      const size_t o = (size_t(sx) * L.T + t) * I + (rg0 + r) * 16 + 4 * g;
      *reinterpret_cast<u32x2*>(L.hs + o) = u32x2{hi[0], hi[1]};
      *reinterpret_cast<u32x2*>(L.hs + plane + o) = u32x2{lo[0], lo[1]};
    }
  }
}

// Prefill shared down: (shared expert, 256 rows of H, 64 tokens) per half
// workgroup; h enters as its bf16 hi and lo parts (two token sources).
__device__ __forceinline__ void shared_down_mx_role(const GemvLayer& L, int b, uint8_t* lds) {
  const int n_rt = (L.H + 255) / 256, n_tt = (L.T + bf::kTok - 1) / bf::kTok;
  int pair, tt;
  bool valid;
  if (!shared_mx_unit(b, L.S * n_rt, n_tt, pair, tt, valid)) return;
  lds += (threadIdx.x / (kWave * 4)) * 4 * bf::kStageBytes;
  const int sx = pair / n_rt, rt = pair % n_rt;
  const int wave = bf::group_wave();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, I = L.I;
  const int nu = I / 32, ngroups = H / 16;
  const int rg0 = rt * 16 + 4 * wave;
  const int t0 = tt * bf::kTok;
  const uint16_t* dm = L.sdown + size_t(sx) * H * I;
  const size_t plane = size_t(L.S) * L.T * I;
  bf::f32x4 acc[bf::kNS][bf::kSub];
  bf::gemm_tile<2>(
      acc,
      [&](int s, int kt) {
        const int rg = min(rg0 + s, ngroups - 1);
        return dm + (size_t(rg) * nu + min(kt, nu - 1)) * 512 + 8 * lane;
      },
      I, lds, [&](int src, int j) {
        return L.hs + src * plane + (size_t(sx) * L.T + min(t0 + j, L.T - 1)) * I;
      });
  if (!valid) return;
#pragma unroll
  for (int u = 0; u < bf::kSub; ++u) {
    const int t = t0 + 16 * u + c;
    if (t >= L.T) continue;
#pragma unroll
    for (int s = 0; s < bf::kNS; ++s) {
      if (rg0 + s >= ngroups) continue;
      *reinterpret_cast<bf::f32x4*>(L.ysh + (size_t(sx) * L.T + t) * H + (rg0 + s) * 16 + 4 * g) =
          acc[s][u];
    }
  }
}

// ------------------------------------------------------------------------
// Prefill roles.

// x rows -> MXFP8 or MXFP4 (L.afmt): thread per 32-element block of the
// padded row (blocks past H get zero codes and exponent 127).
__device__ void quant_x_role(const GemvLayer& L, int b) {
  const int nbq = L.Kq / 32;
  const size_t gb = size_t(b) * kThreads + threadIdx.x;
  if (gb >= size_t(L.T) * nbq) return;
  const int t = int(gb / nbq), kb = int(gb % nbq);
  const bool fp4 = L.afmt == mx::kFmtFp4;
  uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int E = 0;
  if (kb * 32 < L.H) {
    const u32x4* src = reinterpret_cast<const u32x4*>(L.x + size_t(t) * L.H + kb * 32);
    u32x4 v[4];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = src[i];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i][d])), fabsf(bf16_hi(v[i][d]))));
    }
    if (fp4) {
      E = mxfp4_block_exp(amax);
      // element 2 n in the low nibble of byte n: 8 elements per dword
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t c0 = e2m1_rne_sat(__builtin_ldexpf(bf16_lo(v[i][d]), -E));
          const uint32_t c1 = e2m1_rne_sat(__builtin_ldexpf(bf16_hi(v[i][d]), -E));
          words[i] |= (c0 | (c1 << 4)) << (8 * d);
        }
    } else {
      E = mxfp8_block_exp(amax);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t c0 = e4m3_rne_sat(__builtin_ldexpf(bf16_lo(v[i][d]), -E));
          const uint32_t c1 = e4m3_rne_sat(__builtin_ldexpf(bf16_hi(v[i][d]), -E));
          words[2 * i + d / 2] |= (c0 | (c1 << 8)) << (16 * (d % 2));
        }
    }
  }
  if (fp4) {
    *reinterpret_cast<u32x4*>(L.xq + size_t(t) * (L.Kq / 2) + kb * 16) =
        u32x4{words[0], words[1], words[2], words[3]};
  } else {
    u32x4* dst = reinterpret_cast<u32x4*>(L.xq + size_t(t) * L.Kq + kb * 32);
    dst[0] = u32x4{words[0], words[1], words[2], words[3]};
    dst[1] = u32x4{words[4], words[5], words[6], words[7]};
  }
  L.xs[size_t(t) * nbq + mx::scale_pos(kb)] = uint8_t(E + 127);
}

// Token tile ti of the plan: slot, first pair and number of pairs.
struct MxTile {
  int a, p0, mt;
};

// The tile's pair ids (clamped to its last pair) in LDS, so the per-step
// staging addresses come from LDS: a global load there would make every
// staging pass wait for all outstanding loads, the weight prefetch included.
__device__ __forceinline__ void load_tile_pairs(const GemvLayer& L, const MxTile& tt, int* lp) {
  if (threadIdx.x < mx::kTok) lp[threadIdx.x] = L.plan.pairs[tt.p0 + min(int(threadIdx.x), tt.mt - 1)];
  __syncthreads();
}
__device__ __forceinline__ bool mx_tile(const GemvLayer& L, int ti, MxTile& t) {
  if (ti >= L.plan.n_mtiles[0]) return false;
  const int packed = L.plan.mtiles[ti];
  t.a = packed >> 16;
  t.p0 = L.plan.act_off[t.a] + (packed & 0xFFFF) * mx::kTok;
  t.mt = min(mx::kTok, L.plan.act_off[t.a + 1] - t.p0);
  return true;
}

// Block b of a prefill GEMM launch -> (token tile, row tile rt of tiles_r).
// Blocks are dealt to the 8 XCDs round-robin (XCD b % 8), so each XCD takes
// groups of kMxGroup consecutive token tiles and runs every row tile of the
// group, the group's tiles side by side: the row tiles of a token tile read
// its activations from one L2, and consecutive token tiles of one expert
// (one in three experts has several at 4096 tokens) read each weight row
// tile within a few blocks of each other, so all but the first come from L2.
// The launch has 8 kMxGroup ceil(tiles / (8 kMxGroup)) tiles_r blocks.
__device__ __forceinline__ bool mx_unit(const GemvLayer& L, int b, int tiles_r, MxTile& t,
                                        int& rt) {
  const int i = b / 8, rem = i % (kMxGroup * tiles_r);
  rt = rem / kMxGroup;
  return mx_tile(L, kMxGroup * (b % 8 + 8 * (i / (kMxGroup * tiles_r))) + rem % kMxGroup, t);
}

// Prefill gate/up: workgroup (8 waves) = (token tile, 256 rows of I); wave w
// takes row groups 2 w, 2 w + 1 of gate and up (4 A streams) against the
// tile's up to 128 tokens.  Epilogue: h = SiLU(g) * u in fp32, then MXFP8
// (or MXFP4) along I -- the wave's 32 rows are exactly one block per token.
__device__ __forceinline__ void mx_gateup_role(const GemvLayer& L, int b, uint8_t* lds) {
  const int tiles_r = (L.I + kMxRowsGU - 1) / kMxRowsGU;
  MxTile tt;
  int rt;
  if (!mx_unit(L, b, tiles_r, tt, rt)) return;
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, I = L.I;
  const int e = L.plan.active[tt.a];
  const PackedMx pm(I, H);
  const int ngroups = I / 16;
  const int rg0 = rt * (kMxRowsGU / 16) + 2 * wave;
  const uint8_t* rec = record_of(L, e);
  const uint8_t* base[2] = {rec, rec + pm.bytes};
  mx::AStreams st;
  st.nkb = pm.nkb;
  st.nsup = pm.nsup;
  st.lane_code = 16 * lane;
  st.lane_scl = 4 * lane;
#pragma unroll
  for (int s = 0; s < mx::kNS; ++s) {
    // the same in every lane: kept in SGPRs, so each weight load needs only
    // the lane's 32-bit offset
    const int rg = min(rg0 + (s & 1), ngroups - 1);
    st.codes[s] = mx::uniform_gptr(base[s >> 1] + size_t(rg) * pm.nkb * 1024);
    st.scl[s] = mx::uniform_gptr(base[s >> 1] + pm.scale_dword(rg, 0, 0));
  }
  __shared__ int pairs[mx::kTok];
  load_tile_pairs(L, tt, pairs);
  auto tok = [&](int j) { return pairs[j] / L.k; };
  const bool fp4 = L.afmt == mx::kFmtFp4;
  const int xrow = fp4 ? L.Kq / 2 : L.Kq, hrow_b = fp4 ? L.Iq / 2 : L.Iq;  // code row bytes
  mx::f32x4 acc[mx::kNS][mx::kSub];
  auto row = [&](int j) { return uint32_t(tok(j)) * uint32_t(xrow); };
  auto srow = [&](int j) { return uint32_t(tok(j)) * uint32_t(L.Kq / 32); };
  if (fp4)
    mx::gemm_tile<mx::kFmtFp4>(acc, st, pm.nkb4 / 2, lds, tt.mt, L.xq, L.xs, row, srow);
  else
    mx::gemm_tile<mx::kFmtFp8>(acc, st, pm.nkb4 / 2, lds, tt.mt, L.xq, L.xs, row, srow);
  if (rt == tiles_r - 1 && L.Iq > I) {
    // h columns I .. Iq are read by the down GEMM against clamped weight
    // tiles: zero codes with a finite exponent make them contribute 0
    const int pad_bytes = (fp4 ? (L.Iq - I) / 2 : L.Iq - I), hbase = fp4 ? I / 2 : I;
    const int pad16 = pad_bytes / 16, pad_blocks = (L.Iq - I) / 32;
    for (int i = threadIdx.x; i < tt.mt * pad16; i += kMxThreads)
      *reinterpret_cast<u32x4*>(L.hq + size_t(tt.p0 + i / pad16) * hrow_b + hbase +
                                16 * (i % pad16)) = u32x4{0, 0, 0, 0};
    for (int i = threadIdx.x; i < tt.mt * pad_blocks; i += kMxThreads)
      L.hs8[size_t(tt.p0 + i / pad_blocks) * (L.Iq / 32) +
            mx::scale_pos(I / 32 + i % pad_blocks)] = 127;
  }
  if (rg0 >= ngroups) return;  // no rows for this wave (I not a multiple of 128)
  const int r0 = rt * kMxRowsGU + 32 * wave;  // the wave's first row along I
  const int blk = r0 / 32;                      // its MX block
#pragma unroll
  for (int u = 0; u < mx::kSub; ++u) {
    float h[2][4];
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[r][i] = silu(acc[r][u][i]) * acc[2 + r][u][i];
        amax = fmaxf(amax, fabsf(h[r][i]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
    const int E = fp4 ? mxfp4_block_exp(amax) : mxfp8_block_exp(amax);
    const int j = 16 * u + c;
    if (j < tt.mt) {
      const int pos = tt.p0 + j;  // h rows in plan order: a tile's rows are contiguous
      // lane (c, g) holds elements 16 r + 4 g .. + 3 of the wave's 32-row block
      if (fp4) {
        uint8_t* hrow = L.hq + size_t(pos) * hrow_b + r0 / 2;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          uint32_t half = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) half |= e2m1_rne_sat(__builtin_ldexpf(h[r][i], -E)) << (4 * i);
          *reinterpret_cast<uint16_t*>(hrow + 8 * r + 2 * g) = uint16_t(half);
        }
      } else {
        uint8_t* hrow = L.hq + size_t(pos) * hrow_b + r0;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          uint32_t word = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) word |= e4m3_rne_sat(__builtin_ldexpf(h[r][i], -E)) << (8 * i);
          *reinterpret_cast<uint32_t*>(hrow + 16 * r + 4 * g) = word;
        }
      }
      if (g == 0) L.hs8[size_t(pos) * (L.Iq / 32) + mx::scale_pos(blk)] = uint8_t(E + 127);
    }
  }
}

// Prefill down: workgroup (8 waves) = (token tile, 512 rows of H); wave w
// takes row groups 4 w .. 4 w + 3.  Writes fp32 partials per pair (combined
// later).
__device__ __forceinline__ void mx_down_role(const GemvLayer& L, int b, uint8_t* lds) {
  const int tiles_r = (L.H + kMxRowsD - 1) / kMxRowsD;
  MxTile tt;
  int rt;
  if (!mx_unit(L, b, tiles_r, tt, rt)) return;
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, I = L.I;
  const int e = L.plan.active[tt.a];
  const PackedMx pgu(I, H), pd(H, I);
  const int ngroups = H / 16;
  const int rg0 = rt * (kMxRowsD / 16) + 4 * wave;
  const uint8_t* base = record_of(L, e) + 2 * pgu.bytes;
  mx::AStreams st;
  st.nkb = pd.nkb;
  st.nsup = pd.nsup;
  st.lane_code = 16 * lane;
  st.lane_scl = 4 * lane;
#pragma unroll
  for (int s = 0; s < mx::kNS; ++s) {
    const int rg = min(rg0 + s, ngroups - 1);
    st.codes[s] = mx::uniform_gptr(base + size_t(rg) * pd.nkb * 1024);
    st.scl[s] = mx::uniform_gptr(base + pd.scale_dword(rg, 0, 0));
  }
  __shared__ int pairs[mx::kTok];
  load_tile_pairs(L, tt, pairs);
  mx::f32x4 acc[mx::kNS][mx::kSub];
  const bool fp4 = L.afmt == mx::kFmtFp4;
  const int hrow_b = fp4 ? L.Iq / 2 : L.Iq;  // code row bytes
  const uint8_t* hc = L.hq + size_t(tt.p0) * hrow_b;
  const uint8_t* hs = L.hs8 + size_t(tt.p0) * (L.Iq / 32);
  auto row = [&](int j) { return uint32_t(min(j, tt.mt - 1)) * uint32_t(hrow_b); };
  auto srow = [&](int j) { return uint32_t(min(j, tt.mt - 1)) * uint32_t(L.Iq / 32); };
  if (fp4)
    mx::gemm_tile<mx::kFmtFp4>(acc, st, pd.nkb4 / 2, lds, tt.mt, hc, hs, row, srow);
  else
    mx::gemm_tile<mx::kFmtFp8>(acc, st, pd.nkb4 / 2, lds, tt.mt, hc, hs, row, srow);
#pragma unroll
  for (int u = 0; u < mx::kSub; ++u) {
    const int j = 16 * u + c;
    if (j >= tt.mt) continue;
    float* prow = L.part + size_t(pairs[j]) * H;
#pragma unroll
    for (int s = 0; s < mx::kNS; ++s) {
      if (rg0 + s >= ngroups) continue;
      __builtin_nontemporal_store(acc[s][u],
                                  reinterpret_cast<mx::f32x4*>(prow + (rg0 + s) * 16 + 4 * g));
    }
  }
}

// Prefill combine: y[t] = sum_j w[t][j] part[t k + j] + sum_s ysh[s][t]
// (+ residual), rounded once to bf16; one token per workgroup, four outputs
// per thread and step.
static_assert(4 * kThreads == 1024, "combine_chunks counts 1024-column chunks");
__device__ void combine_role(const GemvLayer& L, int b) {
  // workgroup = (token, 4 kThreads columns): one short pass per workgroup
  // streams better than one workgroup looping over a token's row (measured:
  // 392 -> 368 us at 4096 tokens x 7168)
  const int nch = combine_chunks(L.H);
  const int t = b / nch, ch = b - t * nch;
  if (t >= L.T) return;
  const int H = L.H, k = L.k;
  // Every load is unconditional (clamped index, stand-in rows for absent
  // operands) and the values of a group are taken together: a load under a
  // condition would be waited for on its own, one round trip each.
  const float* ysh = L.S > 0 ? L.ysh : L.part;
  const uint16_t* res = L.residual != nullptr ? L.residual : L.x;
  for (int n = ch * 4 * kThreads + 4 * threadIdx.x; n < min(H, (ch + 1) * 4 * kThreads);
       n += 4 * kThreads) {
    mx::f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    mx::f32x4 sv[4];
    u32x2 rv = {0u, 0u};
    for (int j0 = 0; j0 < k; j0 += 16) {
      mx::f32x4 pv[16];
      float wv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const size_t p = size_t(t) * k + min(j0 + j, k - 1);
        pv[j] = __builtin_nontemporal_load(reinterpret_cast<const mx::f32x4*>(L.part + p * H + n));
        wv[j] = L.w[p];
      }
      if (j0 == 0) {
#pragma unroll
        for (int sx = 0; sx < 4; ++sx)
          sv[sx] = *reinterpret_cast<const mx::f32x4*>(
              ysh + (size_t(max(min(sx, L.S - 1), 0)) * L.T + t) * H + n);
        rv = *reinterpret_cast<const u32x2*>(res + size_t(t) * H + n);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(pv[j]), "+v"(wv[j]));
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j0 + j < k)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = fmaf(wv[j], pv[j][i], acc[i]);
    }
#pragma unroll
    for (int sx = 0; sx < 4; ++sx)
      if (sx < L.S)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += sv[sx][i];
    if (L.residual != nullptr) {
      acc[0] += bf16_lo(rv[0]);
      acc[1] += bf16_hi(rv[0]);
      acc[2] += bf16_lo(rv[1]);
      acc[3] += bf16_hi(rv[1]);
    }
    *reinterpret_cast<u32x2*>(L.y + size_t(t) * H + n) =
        u32x2{uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16),
              uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16)};
  }
}

// The top-k workgroup of the router launch (T <= kSelwMaxTokens, the launch's last block) waits
// until every logits workgroup has flagged its logits with this call's epoch, then clears the
// flags for the next call. Only this one workgroup waits, on workgroups that wait on nothing, so
// the others always get to run. The wait is bounded (L.spin_limit polls): if it gives up, the
// workspace status word is set to kWaitGaveUp, which the caller reads with moe_workspace_status,
// and the selection runs on what is there (wrong results, no hang).
__device__ void select_waits(const GemvLayer& L, int n) {
  wait_flags(L, L.lflags, n);
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kThreads) L.lflags[i] = 0;
}

// kRounds: the most tokens per wave (kSelwMaxTokens / kWaves where the
// router launch's top-k can take up to kSelwMaxTokens tokens, else 1), a
// compile-time bound so that the other launches' top-k code is unchanged.
template <bool kCoherent = false, int kRounds = 1>
__device__ void select_role(const GemvLayer& L, const Stage& st, int b) {
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
  // With one top-k workgroup (T <= kSelwMaxTokens; its waves take the
  // tokens in turn) it builds the plan straight from its own selections in
  // LDS: no arrival count, and no round trips through the coherent level for
  // the ids it has just computed.
  const bool single = st.n_select + st.n_selw == 1;
  __shared__ int own_ids[kSelwMaxTokens * 32];
  __shared__ SelectScratch sc[kWaves];
  int id = 0;  // this lane's selected expert (lanes < k of a token's wave)
  const int rounds = single ? min(kRounds, (L.T + kWaves - 1) / kWaves) : 1;
#pragma nounroll
  for (int r = 0; r < kRounds; ++r) {  // one copy of the selection code, not kRounds
    if (r >= rounds) break;  // uniform
    const int t = (single ? r : b) * kWaves + wave;
    if (t < L.T) {
      float w;
      const float* lrow = L.logits + size_t(t) * L.E;
      const size_t ps = size_t(L.T) * L.E;
      if (L.sbias != nullptr) {
        if (L.lsplit == kRouterSplit)
          select_token<kCoherent, kRouterSplit, true>(lrow, ps, L.E, L.k, id, w, sc[wave], L.sbias,
                                                      L.rscale);
        else
          select_token<kCoherent, 1, true>(lrow, 0, L.E, L.k, id, w, sc[wave], L.sbias, L.rscale);
      } else if (L.lsplit == kRouterSplit) {
        select_token<kCoherent, kRouterSplit>(lrow, ps, L.E, L.k, id, w, sc[wave], nullptr,
                                              L.rscale);
      } else {
        select_token<kCoherent>(lrow, 0, L.E, L.k, id, w, sc[wave], nullptr, L.rscale);
      }
      if (lane < L.k) {
        if (single && !L.front) {
          L.ids_out[size_t(t) * L.k + lane] = id;
          L.w_out[size_t(t) * L.k + lane] = w;
          own_ids[t * L.k + lane] = id;
        } else {  // read by other workgroups of this launch (or the next top-k's plan)
          store_coherent(&L.ids_out[size_t(t) * L.k + lane], id);
          store_coherent(&L.w_out[size_t(t) * L.k + lane], w);
        }
      }
    }
  }
  // Direct mode (no plan): only the combine's arrival counters need clearing,
  // before the ids flag: a routed down of the same launch may count once it
  // sees the flag.
  if (st.plan_after_select && L.direct)
    for (int i = threadIdx.x; i < L.n_tiles; i += kThreads) store_coherent(&L.tile_cnt[i], 0);
  if (L.front) {  // ids, weights and counters stored (above): publish the slots' experts
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (wave == 0 && lane < L.k && L.T == 1)
      store_coherent(&L.idtag[lane], (L.epoch & 0xFFFFFFFFFFFFull) << 16 | uint32_t(id));
    if (threadIdx.x == 0) store_coherent(L.idsflag, L.epoch);
  }
  if (!st.plan_after_select || L.direct) return;
  if (single) {
    __syncthreads();
    build_plan([&](int p) { return own_ids[p]; }, L.T * L.k, L.E, L.plan, L.tile_cnt, L.n_tiles);
    return;
  }
  if (!arrive_last(L.sel_cnt, st.n_select)) return;
  const int32_t* ids = L.ids_out;
  build_plan([&](int p) { return load_coherent(ids + p); }, L.T * L.k, L.E, L.plan, L.tile_cnt,
             L.n_tiles);
}

template <bool kFront>
__device__ void routed_down_role(const GemvLayer& L, int a, int tile, uint16_t* hsm) {
  int n_active, e, p0, p1;
  slot_of(L, a, n_active, e, p0, p1);
  if (a >= n_active) return;  // slot beyond this routing's experts
  if constexpr (kFront) {
    routed_down<kDownStagesFront, true>(L, a, e, p0, p1, tile, hsm);
    if (arrive_last(&L.tile_cnt[tile], front_arrivals(L, tile)))
      combine_tile<kFrontDownRows, true>(L, tile);
  } else {
    routed_down<kDownStages, false>(L, a, e, p0, p1, tile, hsm);
    if (arrive_last(&L.tile_cnt[tile], n_active)) combine_tile<kRowsD, false>(L, tile);
  }
}

template <unsigned R, int NCH>
__device__ __forceinline__ void stage_body(const GemvLayer& L, const Stage& st) {
  extern __shared__ u32x4 lds_raw[];
  uint16_t* lds16p = reinterpret_cast<uint16_t*>(lds_raw);
  __shared__ float red[(R & (kRoleSharedGU | kRoleRoutedGU)) ? kWaves * kWave * 8 : 1];
  int b = blockIdx.x;
  if constexpr ((R & kRoleLogits) != 0) {
    if (b < st.n_logits) {
      // the select workgroups of the next launch count their arrivals here
      if (b == 0 && threadIdx.x == 0 && L.sel_cnt != nullptr) L.sel_cnt[0] = 0;
      if (L.lsplit == kRouterSplit)
        router_split_role(L, b, red);
      else
        router_logits_rows<NCH>(L.x, L.wr, L.rbias, L.logits, L.T, L.H, L.E, b, lds_raw);
      if (st.n_selw > 0) {  // logits stored (through the coherent level): flag them
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) store_coherent(&L.lflags[b], L.epoch);
      }
      return;
    }
    b -= st.n_logits;
  }
  if constexpr ((R & kRoleSelect) != 0) {
    if (b < st.n_select) {
      select_role(L, st, b);
      return;
    }
    b -= st.n_select;
  }
  if constexpr ((R & kRolePlan) != 0) {
    if (b < st.n_plan) {
      if (L.direct) {
        for (int i = threadIdx.x; i < L.n_tiles; i += kThreads) L.tile_cnt[i] = 0;
        return;
      }
      const int32_t* ids = L.ids_in;
      build_plan([&](int p) { return ids[p]; }, L.T * L.k, L.E, L.plan, L.tile_cnt,
                 L.n_tiles);
      return;
    }
    b -= st.n_plan;
  }
  if constexpr ((R & kRoleQuantX) != 0) {
    if (b < st.n_xq) {
      quant_x_role(L, b);
      return;
    }
    b -= st.n_xq;
  }
  if constexpr ((R & kRoleMxGateUp) != 0) {
    if (b < st.n_mgu) {
      mx_gateup_role(L, b, reinterpret_cast<uint8_t*>(lds_raw));
      return;
    }
    b -= st.n_mgu;
  }
  if constexpr ((R & kRoleMxDown) != 0) {
    if (b < st.n_mdn) {
      mx_down_role(L, b, reinterpret_cast<uint8_t*>(lds_raw));
      return;
    }
    b -= st.n_mdn;
  }
  if constexpr ((R & kRoleCombine) != 0) {
    if (b < st.n_comb) {
      combine_role(L, b);
      return;
    }
    b -= st.n_comb;
  }
  if constexpr ((R & kRoleRouterMx) != 0) {
    if (b < st.n_rmx) {
      router_mx_role(L, b, reinterpret_cast<uint8_t*>(lds_raw));
      return;
    }
    b -= st.n_rmx;
  }
  if constexpr ((R & kRoleSharedGUMx) != 0) {
    if (b < st.n_sgmx) {
      shared_gu_mx_role(L, b, reinterpret_cast<uint8_t*>(lds_raw));
      return;
    }
    b -= st.n_sgmx;
  }
  if constexpr ((R & kRoleSharedDownMx) != 0) {
    if (b < st.n_sdmx) {
      shared_down_mx_role(L, b, reinterpret_cast<uint8_t*>(lds_raw));
      return;
    }
    b -= st.n_sdmx;
  }
  const int gu_tiles = L.I / 32;
  // The shared roles: one workgroup per (expert, row group or tile, pass of
  // tokens), the passes of one row range on one XCD (xcd_split), where the
  // first to load the weights leaves them in L2 for the others.
  if constexpr ((R & kRoleSharedGU) != 0) {
    if (b < st.n_sgu) {
      const int rows = L.I / 16, n_pass = (L.T + kCols - 1) / kCols;
      int unit, pass;
      if (!xcd_split(b, L.S * rows, n_pass, unit, pass)) return;
      const int p0 = pass * kCols, p1 = min(L.T, p0 + kCols);
      if (n_pass > 1) shared_gateup<true>(L, unit / rows, unit % rows, red, p0, p1);
      else shared_gateup<false>(L, unit / rows, unit % rows, red, p0, p1);
      return;
    }
    b -= st.n_sgu;
  }
  if constexpr ((R & kRoleSharedDown) != 0) {
    if (b < st.n_sdn) {
      const int n_pass = (L.T + kCols / 2 - 1) / (kCols / 2);
      int unit, pass;
      if (!xcd_split(b, L.S * L.n_stiles, n_pass, unit, pass)) return;
      const int p0 = pass * (kCols / 2), p1 = min(L.T, p0 + kCols / 2);
      if (n_pass > 1) shared_down<true>(L, unit / L.n_stiles, unit % L.n_stiles, p0, p1);
      else shared_down<false>(L, unit / L.n_stiles, unit % L.n_stiles, p0, p1);
      return;
    }
    b -= st.n_sdn;
  }
  if constexpr ((R & kRoleRoutedGU) != 0) {
    if (b < st.n_rgu) {
      routed_gateup(L, b / gu_tiles, b % gu_tiles, lds16p, red);
      return;
    }
    b -= st.n_rgu;
  }
  if constexpr ((R & kRoleRoutedDown) != 0) {
    if (b < st.n_rdn) {
      routed_down_role<false>(L, b / L.n_tiles, b % L.n_tiles, lds16p);
      return;
    }
    b -= st.n_rdn;
  }
  if constexpr ((R & kRoleSelectWait) != 0) {  // last: it waits on the blocks before it
    if (b < st.n_selw) {
      select_waits(L, st.n_logits);
      select_role<true, kSelwMaxTokens / kWaves>(L, st, 0);
    }
  }
}

// One-token decode: every workgroup role of the layer in one launch, in
// this block order: router logits (each flags its logits), shared gate/up
// (each flags its h rows), the top-k (waits for the logits flags, publishes
// each slot's expert), routed gate/up (waits for its slot's expert, flags its
// h rows), routed down (waits for its slot's expert and gate/up flags,
// counts its tile's arrival), shared down (waits for its shared expert's
// gate/up flags, counts its tile's arrival); the last arriver of a tile
// combines it.  A workgroup only waits for blocks with lower indices, which
// the dispatcher hands out first (in order on every XCD), so the
// lowest-indexed unfinished block can always run to its end: every wait
// ends; each is bounded besides (wait_flags).  The routed streams start as
// soon as the top-k is done, while the shared experts still stream, and the
// routed down starts while the gate/up of later slots still streams: no
// launch boundary drains the machine between them.  Measured against other
// block orders and tile sizes (routed gate/up first, shared down before the
// routed down, 64-row gate/up or 128/512-row down tiles): all slower.
template <int NCH>
__device__ __forceinline__ void front_body(const GemvLayer& L, const Stage& st) {
  extern __shared__ u32x4 lds_raw[];
  uint16_t* lds16p = reinterpret_cast<uint16_t*>(lds_raw);
  __shared__ float red[kWaves * kWave * 8];
  const int sgu_rows = L.I / 16, gu_tiles = L.I / 32;
  int b = blockIdx.x;
  // router logits
  if (b < st.n_logits) {
    if (b == 0 && threadIdx.x == 0 && L.sel_cnt != nullptr) L.sel_cnt[0] = 0;
    router_logits_rows<NCH>(L.x, L.wr, L.rbias, L.logits, L.T, L.H, L.E, b, lds_raw);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) store_coherent(&L.lflags[b], L.epoch);
    return;
  }
  b -= st.n_logits;
  // shared gate/up
  if (b < st.n_sgu) {
    shared_gateup<false, kSharedStagesFront>(L, b / sgu_rows, b % sgu_rows, red);
    return;
  }
  b -= st.n_sgu;
  // top-k
  if (b < st.n_selw) {
    select_waits(L, st.n_logits);
    select_role<true>(L, st, 0);
    return;
  }
  b -= st.n_selw;
  // routed gate/up
  if (b < st.n_rgu) {  // waits for its slot's expert (slot_of)
    routed_gateup<true>(L, b / gu_tiles, b % gu_tiles, lds16p, red);
    return;
  }
  b -= st.n_rgu;
  // routed down
  if (b < st.n_rdn) {  // waits for its slot's gate/up flags
    const int nft = (L.H + kFrontDownRows - 1) / kFrontDownRows;
    routed_down_role<true>(L, b / nft, b % nft, lds16p);
    return;
  }
  b -= st.n_rdn;
  // shared down
  if (b < st.n_sdn) {
    shared_down_front(L, b / L.n_stiles, b % L.n_stiles, lds16p);
  }
}

// The launches, named for what they run.
template <int NCH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kFrontWaves))) void
moe_decode_front(GemvLayer L, Stage st) {
  front_body<NCH>(L, st);
}
template <int NCH>
__global__ __launch_bounds__(kThreads) void moe_router_shared_gateup(GemvLayer L, Stage st) {
  stage_body<kRoleLogits | kRoleSharedGU | kRoleSelectWait, NCH>(L, st);
}
__global__ __launch_bounds__(kThreads) void moe_select_shared_down(GemvLayer L, Stage st) {
  stage_body<kRoleSelect | kRoleSharedDown, 0>(L, st);
}
__global__ __launch_bounds__(kThreads) void moe_plan_shared_gateup(GemvLayer L, Stage st) {
  stage_body<kRolePlan | kRoleSharedGU, 0>(L, st);
}
__global__ __launch_bounds__(kThreads) void moe_routed_gateup(GemvLayer L, Stage st) {
  stage_body<kRoleSharedDown | kRoleRoutedGU, 0>(L, st);
}
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void
moe_routed_down_combine(GemvLayer L, Stage st) {
  stage_body<kRoleRoutedDown, 0>(L, st);
}
__global__ __launch_bounds__(kThreads) void moe_plan_quant_shared_gateup(GemvLayer L, Stage st) {
  stage_body<kRolePlan | kRoleQuantX | kRoleSharedGU, 0>(L, st);
}
__global__ __launch_bounds__(kThreads) void moe_router_mx_quant(GemvLayer L, Stage st) {
  stage_body<kRoleQuantX | kRoleRouterMx, 0>(L, st);
}
__global__ __launch_bounds__(kMxThreads) void moe_mx_gateup(GemvLayer L, Stage st) {
  stage_body<kRoleMxGateUp | kRoleSharedGUMx, 0>(L, st);
}
__global__ __launch_bounds__(kMxThreads) void moe_mx_down(GemvLayer L, Stage st) {
  stage_body<kRoleMxDown | kRoleSharedDownMx, 0>(L, st);
}
__global__ __launch_bounds__(kThreads) void moe_combine(GemvLayer L, Stage st) {
  stage_body<kRoleCombine, 0>(L, st);
}

int tokens_per_pass(int T, int row_bytes, int budget) {
  const int t = budget / row_bytes;
  return max(1, min(min(t, kCols), T));
}

}  // namespace

static_assert(kThreads == kPlanThreads, "the plan builder runs on one stage workgroup");

hipError_t launch_stage(StageKind kind, GemvLayer L, Stage st, hipStream_t stream) {
  L.n_tiles = (L.H + kRowsD - 1) / kRowsD;
  L.n_stiles = (L.H + kRowsSD - 1) / kRowsSD;
  const int xrow = pad_k(L.H) + 8, hrow = pad_k(L.I) + 8;  // staged row lengths
  L.mtp_gu = tokens_per_pass(L.T, xrow * 2, kLdsBudgetGU);
  L.mtp_d = min(tokens_per_pass(L.T, hrow * 4, kLdsBudget), kCols / 2);  // hi + lo: two B columns per token
  size_t lds = 0;
  if (st.n_logits > 0) lds = max(lds, size_t(kRouterTokens) * L.H * 2);
  if (st.n_rgu > 0) lds = max(lds, size_t(L.mtp_gu) * xrow * 2);
  if (st.n_rdn > 0) lds = max(lds, size_t(L.mtp_d) * hrow * 4);
  if (st.n_rmx > 0) lds = max(lds, size_t(2 * bf::kStageBytes));
  if (st.n_sgmx > 0) lds = max(lds, size_t(2 * 2 * bf::kStageBytes));  // two halves
  if (st.n_sdmx > 0) lds = max(lds, size_t(2 * 4 * bf::kStageBytes));
  const int wgs = st.n_logits + st.n_select + st.n_plan + st.n_sgu + st.n_sdn + st.n_rgu +
                  st.n_rdn + st.n_xq + st.n_mgu + st.n_mdn + st.n_comb + st.n_rmx + st.n_sgmx +
                  st.n_sdmx + st.n_selw;
  if (wgs <= 0) return hipSuccess;
  if (st.n_mgu > 0 || st.n_mdn > 0)
    lds = max(lds, size_t(L.afmt == mx::kFmtFp4 ? mx::lds_bytes<mx::kFmtFp4>()
                                                 : mx::lds_bytes<mx::kFmtFp8>()));
  const bool mx8 = kind == StageKind::MxGateUp || kind == StageKind::MxDown;
  const dim3 grid(wgs), block(mx8 ? kMxThreads : kThreads);
  const LaunchEvents ev = next_launch_events();
  switch (kind) {
    case StageKind::RouterSharedGateUp: {
      const int per_lane = (L.H / 8 + kWave - 1) / kWave;
      if (per_lane <= 4)
        launch_timed(ev, moe_router_shared_gateup<4>, grid, block, lds, stream, L, st);
      else if (per_lane <= 8)
        launch_timed(ev, moe_router_shared_gateup<8>, grid, block, lds, stream, L, st);
      else
        launch_timed(ev, moe_router_shared_gateup<16>, grid, block, lds, stream, L, st);
      break;
    }
    case StageKind::DecodeFront: {
      const int per_lane = (L.H / 8 + kWave - 1) / kWave;
      if (per_lane <= 4)
        launch_timed(ev, moe_decode_front<4>, grid, block, lds, stream, L, st);
      else if (per_lane <= 8)
        launch_timed(ev, moe_decode_front<8>, grid, block, lds, stream, L, st);
      else
        launch_timed(ev, moe_decode_front<16>, grid, block, lds, stream, L, st);
      break;
    }

    case StageKind::SelectSharedDown:
      launch_timed(ev, moe_select_shared_down, grid, block, lds, stream, L, st);
      break;
    case StageKind::PlanSharedGateUp:
      launch_timed(ev, moe_plan_shared_gateup, grid, block, lds, stream, L, st);
      break;
    case StageKind::RoutedGateUp:
      launch_timed(ev, moe_routed_gateup, grid, block, lds, stream, L, st);
      break;
    case StageKind::RoutedDownCombine:
      launch_timed(ev, moe_routed_down_combine, grid, block, lds, stream, L, st);
      break;
    case StageKind::PlanQuantSharedGateUp:
      launch_timed(ev, moe_plan_quant_shared_gateup, grid, block, lds, stream, L, st);
      break;
    case StageKind::RouterMxQuant:
      launch_timed(ev, moe_router_mx_quant, grid, block, lds, stream, L, st);
      break;
    case StageKind::MxGateUp:
      launch_timed(ev, moe_mx_gateup, grid, block, lds, stream, L, st);
      break;
    case StageKind::MxDown:
      launch_timed(ev, moe_mx_down, grid, block, lds, stream, L, st);
      break;
    case StageKind::Combine:
      launch_timed(ev, moe_combine, grid, block, lds, stream, L, st);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
