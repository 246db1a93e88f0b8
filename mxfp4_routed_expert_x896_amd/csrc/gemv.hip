// Decode-path expert kernels on the matrix cores: dequant-fused MXFP4
// gate/up and down projections for the routed experts, the bf16 shared
// experts, and the weighted combine.
//
// Deltafin README ("An experiment in running Kimi K3 ..."), "Techniques /
// Compute": the MXFP4 weights are decoded inside the product instead of
// being dequantised to a temporary first; the Deltafin explainer
// (bhfrc.com), section 6.2, gives the reason (a separate pass costs memory
// and another trip through memory bandwidth).  Here a weight never exists in
// dequantised form outside registers.  Each lane loads 16 bytes of codes --
// one whole 32-element block of one row, so one E8M0 exponent -- converts
// them with v_cvt_scalef32_pk_bf16_fp4 (the block exponent applied in the
// convert; exact, since an E2M1 value times a power of two is a bf16,
// subnormals included) and feeds them as the A operand of
// v_mfma_f32_16x16x32_bf16.  The tokens routed to the expert are the B
// columns (up to 16 per pass), accumulation is fp32.  At batch 1 only one B
// column is live: the matrix core is used to take the multiply-accumulate
// off the vector ALU (one convert per code byte remains), which is what
// lets the weight stream run near the HBM roof; batched decode then reuses
// every converted weight for all tokens of the expert at no extra cost.
//
// Operand mapping (wave64, lane l: g = l / 16, c = l % 16): weights are
// read in the MFMA-tiled layout written by pack.hip, so for super-step kb a
// wave loads one 1088-byte tile: lane l gets block bi = 4 kb + g of row
// r0 + c (16 contiguous bytes of a 1 KiB contiguous read) and its scale
// byte.  MFMA step s (0..3) takes elements 8 s .. 8 s + 7 of that block,
// i.e. contraction index K = 32 bi + 8 s + j; the B lane (g, c) supplies the
// same K indices of token c.  The 16 x 16 fp32 result leaves rows 4 g + i
// (i = 0..3) of token c in lane (g, c).  bf16 (shared) matrices use 1 KiB
// tiles of 16 rows x 32 columns, lane l holding columns 8 g .. 8 g + 7.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsD = 64;        // down rows per workgroup (16 per wave)
constexpr int kCols = 16;         // B columns of one MFMA: at most 16 tokens per pass
constexpr int kLdsBudget = 32768;  // bytes of staged activations per workgroup

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ f32x4_t mfma(const u32x4& a, const u32x4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32 -> bf16 hi + bf16 lo with hi + lo = v to about 2^-17 relative.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(v);
  lo = f32_to_bf16(v - bf16_to_f32(hi));
}

// Partials cross workgroups (and XCDs, whose L2s are private): they are
// stored and re-read with device-scope atomic accesses, which the compiler
// emits as write-through stores and L2-bypassing loads, instead of fencing
// (a device-scope fence writes back and invalidates the whole L2).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stage the bf16 rows of mt tokens into LDS rows of `stride` elements:
// dst[j][0..K) = src(j)[0..K); sources via the callback src(j).
template <typename Src>
__device__ __forceinline__ void stage_rows(uint16_t* dst, int stride, int mt, int K, Src src) {
  const int nch = K / 8;
  for (int i = threadIdx.x; i < mt * nch; i += kThreads) {
    const int j = i / nch, q = i % nch;
    *reinterpret_cast<u32x4*>(dst + j * stride + q * 8) = ld16(src(j) + q * 8);
  }
}

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ------------------------------------------------------------------------
// Gate/up.  Workgroup = (contributor, 32 rows): wave w takes row group
// w / 2 of the tile and half w % 2 of the contraction; the halves meet in
// LDS.  The tokens' x rows are staged in LDS (B operand), mtp at a time.
// Weight tiles are double-buffered: the loads of super-step kq + 1 are in
// flight while super-step kq is converted and multiplied.

struct GuTiles {
  u32x4 g[4], u[4];
  uint32_t sg, su;
};

__device__ __forceinline__ void load_gu(GuTiles& t, const uint8_t* gcodes, const uint8_t* ucodes,
                                        const uint8_t* gscl, const uint8_t* uscl, int kq, int nkb,
                                        int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kb = 4 * kq + j;
    t.g[j] = kb < nkb ? ld_nt(gcodes + size_t(kb) * 1024 + 16 * lane) : u32x4{0, 0, 0, 0};
    t.u[j] = kb < nkb ? ld_nt(ucodes + size_t(kb) * 1024 + 16 * lane) : u32x4{0, 0, 0, 0};
  }
  t.sg = *reinterpret_cast<const uint32_t*>(gscl + 4 * kq);
  t.su = *reinterpret_cast<const uint32_t*>(uscl + 4 * kq);
}

__device__ __forceinline__ void mma_gu(const GuTiles& t, const uint16_t* xrow, int kq, int nb,
                                       int g, f32x4_t& ag, f32x4_t& au) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bi = 16 * kq + 4 * j + g;
    const float sg = e8m0_to_f32((t.sg >> (8 * j)) & 0xFFu);
    const float su = e8m0_to_f32((t.su >> (8 * j)) & 0xFFu);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 bx = bi < nb ? lds16(xrow + bi * 32 + 8 * s) : u32x4{0, 0, 0, 0};
      ag = mfma(fp4x8_scaled(t.g[j][s], sg), bx, ag);
      au = mfma(fp4x8_scaled(t.u[j][s], su), bx, au);
    }
  }
}

// Adds the partner half's tiles (wave w ^ 1) into waves with even index.
__device__ __forceinline__ void join_halves(f32x4_t& a, f32x4_t& b, float* red) {
  const int wave = threadIdx.x / kWave;
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

__device__ void routed_gateup(const GemvLayer& L, int a, int tile, uint16_t* xs, float* red) {
  if (a >= L.plan.n_active[0]) return;
  const int e = L.plan.active[a];
  const int p0 = L.plan.act_off[a];
  const int p1 = L.plan.act_off[a + 1];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, I = L.I;
  const PackedMx pm(I, H);
  const int nkq = pm.nkb4 / 4;
  const int kqh = (nkq + 1) / 2;
  const int kq0 = (wave & 1) * kqh, kq1 = min(kq0 + kqh, nkq);
  const int rg = tile * 2 + wave / 2;
  const uint8_t* gbase = L.experts + size_t(e) * L.stride;
  const uint8_t* ubase = gbase + pm.bytes;
  const uint8_t* gcodes = gbase + size_t(rg) * pm.nkb * 1024;
  const uint8_t* ucodes = ubase + size_t(rg) * pm.nkb * 1024;
  const uint8_t* gscl = gbase + pm.code_bytes + (size_t(rg) * 64 + lane) * pm.nkb4;
  const uint8_t* uscl = ubase + pm.code_bytes + (size_t(rg) * 64 + lane) * pm.nkb4;
  const int xstride = H + 8;
  uint16_t* hhi = L.h;
  uint16_t* hlo = L.h + size_t(L.T) * L.k * I;

  for (int t0 = p0; t0 < p1; t0 += L.mtp_gu) {
    const int mt = min(L.mtp_gu, p1 - t0);
    GuTiles cur, nxt;
    if (kq0 < kq1) load_gu(cur, gcodes, ucodes, gscl, uscl, kq0, pm.nkb, lane);
    __syncthreads();
    stage_rows(xs, xstride, mt, H, [&](int j) {
      return L.x + size_t(min(L.plan.pairs[t0 + j] / L.k, L.T - 1)) * H;
    });
    __syncthreads();
    const uint16_t* xrow = xs + (c < mt ? c : 0) * xstride;
    f32x4_t ag = {0.0f, 0.0f, 0.0f, 0.0f}, au = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int kq = kq0; kq < kq1; ++kq) {
      if (kq + 1 < kq1) load_gu(nxt, gcodes, ucodes, gscl, uscl, kq + 1, pm.nkb, lane);
      mma_gu(cur, xrow, kq, pm.nb, g, ag, au);
      cur = nxt;
    }
    join_halves(ag, au, red);
    if (!(wave & 1) && c < mt) {
      const int pair = L.plan.pairs[t0 + c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t hi, lo;
        split_bf16(silu(ag[i]) * au[i], hi, lo);
        const size_t o = size_t(pair) * I + rg * 16 + 4 * g + i;
        hhi[o] = hi;
        hlo[o] = lo;
      }
    }
  }
}

// Shared gate/up (bf16): 1 KiB tiles of 16 rows x 32 columns are the A
// operand as loaded; four tiles per super-step, double-buffered.
__device__ void shared_gateup(const GemvLayer& L, int sx, int tile, uint16_t* xs, float* red) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int H = L.H, I = L.I;
  const int nu = H / 32;
  const int nq = (nu + 3) / 4;
  const int qh = (nq + 1) / 2;
  const int q0 = (wave & 1) * qh, q1 = min(q0 + qh, nq);
  const int rg = tile * 2 + wave / 2;
  const uint16_t* gt = L.sgate + sx * (size_t(I) * H) + size_t(rg) * nu * 512;
  const uint16_t* ut = L.sup + sx * (size_t(I) * H) + size_t(rg) * nu * 512;
  const int xstride = H + 8;
  const size_t plane = size_t(L.S) * L.T * I;
  auto load = [&](u32x4 (&wg)[4], u32x4 (&wu)[4], int q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = 4 * q + j;
      wg[j] = u < nu ? ld_nt(gt + size_t(u) * 512 + 8 * lane) : u32x4{0, 0, 0, 0};
      wu[j] = u < nu ? ld_nt(ut + size_t(u) * 512 + 8 * lane) : u32x4{0, 0, 0, 0};
    }
  };
  for (int t0 = 0; t0 < L.T; t0 += L.mtp_gu) {
    const int mt = min(L.mtp_gu, L.T - t0);
    u32x4 cg[4], cu[4], ng[4], nu4[4];
    if (q0 < q1) load(cg, cu, q0);
    __syncthreads();
    stage_rows(xs, xstride, mt, H, [&](int j) { return L.x + size_t(t0 + j) * H; });
    __syncthreads();
    const uint16_t* xrow = xs + (c < mt ? c : 0) * xstride;
    f32x4_t ag = {0.0f, 0.0f, 0.0f, 0.0f}, au = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int q = q0; q < q1; ++q) {
      if (q + 1 < q1) load(ng, nu4, q + 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int u = 4 * q + j;
        const u32x4 bx = u < nu ? lds16(xrow + u * 32 + 8 * g) : u32x4{0, 0, 0, 0};
        ag = mfma(cg[j], bx, ag);
        au = mfma(cu[j], bx, au);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cg[j] = ng[j];
        cu[j] = nu4[j];
      }
    }
    join_halves(ag, au, red);
    if (!(wave & 1) && c < mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t hi, lo;
        split_bf16(silu(ag[i]) * au[i], hi, lo);
        const size_t o = (size_t(sx) * L.T + t0 + c) * I + rg * 16 + 4 * g + i;
        L.hs[o] = hi;
        L.hs[plane + o] = lo;
      }
    }
  }
}

// Grid: [S * I / 32 shared tiles] then [max_active * I / 32 routed tiles].
__global__ __launch_bounds__(kThreads) void gateup_kernel(GemvLayer L) {
  extern __shared__ u32x4 lds_raw[];
  __shared__ float red[kWaves * kWave * 8];
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds_raw);
  const int tiles = L.I / 32;
  const int shared_wgs = L.S * tiles;
  const int b = blockIdx.x;
  if (b < shared_wgs)
    shared_gateup(L, b / tiles, b % tiles, xs, red);
  else
    routed_gateup(L, (b - shared_wgs) / tiles, (b - shared_wgs) % tiles, xs, red);
}

// ------------------------------------------------------------------------
// Down projections and the combine.  Workgroups are (contributor, tile of
// kRowsD output rows, 16 per wave); contributors are the active experts
// (MXFP4) and the shared experts (bf16).  h enters as bf16 hi + lo, staged
// in LDS, two MFMAs per step.  Each contributor writes fp32 partials for
// its rows and tokens; the last workgroup to finish a tile (device-scope
// counter, zeroed by the plan kernel of the same call) sums the tile's
// partials in a fixed order -- routed slots j = 0..k-1 weighted by w, then
// shared experts, then the residual -- and writes the bf16 output.  The sum
// order does not depend on which workgroup arrives last, so the output is
// deterministic.

struct DnTiles {
  u32x4 w[4];
  uint32_t sc;
};

__device__ void routed_down(const GemvLayer& L, int a, int tile, uint16_t* hsm) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int rg = tile * (kRowsD / 16) + wave;
  const bool live = rg < L.H / 16;  // ragged last tile
  const int e = L.plan.active[a];
  const int p0 = L.plan.act_off[a];
  const int p1 = L.plan.act_off[a + 1];
  const int H = L.H, I = L.I;
  const PackedMx pgu(I, H), pd(H, I);
  const int nkq = pd.nkb4 / 4;
  const uint8_t* base = L.experts + size_t(e) * L.stride + 2 * pgu.bytes;
  const uint8_t* codes = base + size_t(live ? rg : 0) * pd.nkb * 1024;
  const uint8_t* scl = base + pd.code_bytes + (size_t(live ? rg : 0) * 64 + lane) * pd.nkb4;
  const int hstride = I + 8;
  uint16_t* hs_hi = hsm;
  uint16_t* hs_lo = hsm + L.mtp_d * hstride;
  const uint16_t* hhi = L.h;
  const uint16_t* hlo = L.h + size_t(L.T) * L.k * I;
  auto load = [&](DnTiles& t, int kq) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = 4 * kq + j;
      t.w[j] = kb < pd.nkb ? ld_nt(codes + size_t(kb) * 1024 + 16 * lane) : u32x4{0, 0, 0, 0};
    }
    t.sc = *reinterpret_cast<const uint32_t*>(scl + 4 * kq);
  };

  for (int t0 = p0; t0 < p1; t0 += L.mtp_d) {
    const int mt = min(L.mtp_d, p1 - t0);
    DnTiles cur, nxt;
    if (live) load(cur, 0);
    __syncthreads();
    stage_rows(hs_hi, hstride, mt, I,
               [&](int j) { return hhi + size_t(L.plan.pairs[t0 + j]) * I; });
    stage_rows(hs_lo, hstride, mt, I,
               [&](int j) { return hlo + size_t(L.plan.pairs[t0 + j]) * I; });
    __syncthreads();
    if (!live) continue;
    const uint16_t* bh = hs_hi + (c < mt ? c : 0) * hstride;
    const uint16_t* bl = hs_lo + (c < mt ? c : 0) * hstride;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int kq = 0; kq < nkq; ++kq) {
      if (kq + 1 < nkq) load(nxt, kq + 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bi = 16 * kq + 4 * j + g;
        const float sd = e8m0_to_f32((cur.sc >> (8 * j)) & 0xFFu);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 aw = fp4x8_scaled(cur.w[j][s], sd);
          const u32x4 vh = bi < pd.nb ? lds16(bh + bi * 32 + 8 * s) : u32x4{0, 0, 0, 0};
          const u32x4 vl = bi < pd.nb ? lds16(bl + bi * 32 + 8 * s) : u32x4{0, 0, 0, 0};
          acc = mfma(aw, vh, acc);
          acc = mfma(aw, vl, acc);
        }
      }
      cur = nxt;
    }
    if (c < mt) {
      const int pair = L.plan.pairs[t0 + c];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_coherent(&L.part[size_t(pair) * H + rg * 16 + 4 * g + i], acc[i]);
    }
  }
}

__device__ void shared_down(const GemvLayer& L, int sx, int tile, uint16_t* hsm) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int rg = tile * (kRowsD / 16) + wave;
  const bool live = rg < L.H / 16;
  const int H = L.H, I = L.I;
  const int nu = I / 32;
  const int nq = (nu + 3) / 4;
  const uint16_t* dt = L.sdown + sx * (size_t(H) * I) + size_t(live ? rg : 0) * nu * 512;
  const int hstride = I + 8;
  uint16_t* hs_hi = hsm;
  uint16_t* hs_lo = hsm + L.mtp_d * hstride;
  const size_t plane = size_t(L.S) * L.T * I;
  auto load = [&](u32x4 (&w)[4], int q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = 4 * q + j;
      w[j] = u < nu ? ld_nt(dt + size_t(u) * 512 + 8 * lane) : u32x4{0, 0, 0, 0};
    }
  };
  for (int t0 = 0; t0 < L.T; t0 += L.mtp_d) {
    const int mt = min(L.mtp_d, L.T - t0);
    u32x4 cw[4], nw[4];
    if (live) load(cw, 0);
    __syncthreads();
    stage_rows(hs_hi, hstride, mt, I,
               [&](int j) { return L.hs + (size_t(sx) * L.T + t0 + j) * I; });
    stage_rows(hs_lo, hstride, mt, I,
               [&](int j) { return L.hs + plane + (size_t(sx) * L.T + t0 + j) * I; });
    __syncthreads();
    if (!live) continue;
    const uint16_t* bh = hs_hi + (c < mt ? c : 0) * hstride;
    const uint16_t* bl = hs_lo + (c < mt ? c : 0) * hstride;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int q = 0; q < nq; ++q) {
      if (q + 1 < nq) load(nw, q + 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int u = 4 * q + j;
        const u32x4 vh = u < nu ? lds16(bh + u * 32 + 8 * g) : u32x4{0, 0, 0, 0};
        const u32x4 vl = u < nu ? lds16(bl + u * 32 + 8 * g) : u32x4{0, 0, 0, 0};
        acc = mfma(cw[j], vh, acc);
        acc = mfma(cw[j], vl, acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) cw[j] = nw[j];
    }
    if (c < mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_coherent(&L.ysh[(size_t(sx) * L.T + t0 + c) * H + rg * 16 + 4 * g + i], acc[i]);
    }
  }
}

// The last contributor of a tile sums its partials into the bf16 output.
// All of a token's partial loads are issued before the first add, so the
// tail costs one memory round trip, not k of them.
__device__ void combine_tile(const GemvLayer& L, int tile) {
  const int H = L.H;
  const int n_out = L.T * kRowsD;
  for (int idx = threadIdx.x; idx < n_out; idx += kThreads) {
    const int t = idx / kRowsD;
    const int n = tile * kRowsD + idx % kRowsD;
    if (n >= H) continue;
    float pv[32], wv[32], sv[4];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const size_t p = size_t(t) * L.k + j;
      pv[j] = j < L.k ? load_coherent(&L.part[p * H + n]) : 0.0f;
      wv[j] = j < L.k ? L.w[p] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sv[s] = s < L.S ? load_coherent(&L.ysh[(size_t(s) * L.T + t) * H + n]) : 0.0f;
    const float r = L.residual != nullptr ? bf16_to_f32(L.residual[size_t(t) * H + n]) : 0.0f;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if (j < L.k) acc = fmaf(wv[j], pv[j], acc);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (s < L.S) acc += sv[s];
    if (L.residual != nullptr) acc += r;
    L.y[size_t(t) * H + n] = f32_to_bf16(acc);
  }
}

// Grid: [S * tiles shared] then [max_active * tiles routed]; tiles =
// ceil(H / kRowsD), the last one ragged.
__global__ __launch_bounds__(kThreads) void down_kernel(GemvLayer L) {
  extern __shared__ u32x4 lds_raw[];
  uint16_t* hsm = reinterpret_cast<uint16_t*>(lds_raw);
  __shared__ int last;
  const int tiles = (L.H + kRowsD - 1) / kRowsD;
  const int shared_wgs = L.S * tiles;
  const int b = blockIdx.x;
  const int n_active = L.plan.n_active[0];
  int tile;
  if (b < shared_wgs) {
    tile = b % tiles;
    shared_down(L, b / tiles, tile, hsm);
  } else {
    const int a = (b - shared_wgs) / tiles;
    tile = (b - shared_wgs) % tiles;
    if (a >= n_active) return;  // not a contributor
    routed_down(L, a, tile, hsm);
  }
  // Partials were written through to the device-coherent level; wait for
  // every store of the workgroup to complete before counting this
  // contribution, so a workgroup that sees the final count also sees them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev =
        __hip_atomic_fetch_add(&L.tile_cnt[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == n_active + L.S - 1;
  }
  __syncthreads();
  if (last) combine_tile(L, tile);
}

}  // namespace

int tokens_per_pass(int T, int row_bytes) {
  const int t = kLdsBudget / row_bytes;
  return max(1, min(min(t, kCols), T));
}

hipError_t launch_gateup(GemvLayer L, hipStream_t stream) {
  L.mtp_gu = tokens_per_pass(L.T, (L.H + 8) * 2);
  const size_t lds = size_t(L.mtp_gu) * (L.H + 8) * 2;
  const int wgs = (L.S + L.max_active) * (L.I / 32);
  hipLaunchKernelGGL(gateup_kernel, dim3(wgs), dim3(kThreads), lds, stream, L);
  return hipGetLastError();
}

hipError_t launch_down(GemvLayer L, hipStream_t stream) {
  L.mtp_d = tokens_per_pass(L.T, (L.I + 8) * 4);
  const size_t lds = size_t(L.mtp_d) * (L.I + 8) * 4;
  const int wgs = (L.S + L.max_active) * ((L.H + kRowsD - 1) / kRowsD);
  hipLaunchKernelGGL(down_kernel, dim3(wgs), dim3(kThreads), lds, stream, L);
  return hipGetLastError();
}

}  // namespace moe
