// Decode-path expert kernels: dequant-fused MXFP4 GEMV for the routed
// experts, bf16 GEMV for the shared experts, and the weighted combine.
//
// Deltafin README ("An experiment in running Kimi K3 ..."), "Techniques /
// Compute": the MXFP4 weights are decoded inside the product rather than
// dequantised to a temporary first; the Deltafin explainer (bhfrc.com),
// section 6.2, gives the reason: a separate dequantisation pass costs
// memory and another trip through memory bandwidth.  Here a weight never
// exists in dequantised form outside registers: each 16-byte chunk of codes
// (one 32-element scale block) is converted to bf16 pairs with
// v_cvt_scalef32_pk_bf16_fp4 and multiplied into the token with
// v_dot2_f32_bf16; the block's E8M0 exponent scales the block's fp32 partial.
//
// Mapping (gfx950, wave64): one wave owns one weight row at a time; lane l
// reads chunks c = l, l + 64, ... so every load instruction covers 1 KiB of
// contiguous codes; the activations for those chunks stay in registers
// across all rows of the workgroup.  Gate and up rows with the same index are
// processed together so SiLU(g) * u is formed before anything is written.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsGU = 16;   // routed gate/up rows per workgroup
constexpr int kRowsGUS = 4;   // shared gate/up rows per workgroup
constexpr int kRowsD = 32;    // routed down rows per workgroup
constexpr int kRowsDS = 16;   // shared down rows per workgroup
constexpr int kSharedTokens = 2;  // tokens per LDS pass in the shared gate/up

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 32 E2M1 codes (one scale block) against 32 bf16 activations.
__device__ __forceinline__ float block_dot_bf16(const u32x4& codes, const uint32_t* xv, float acc) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = codes[d];
    acc = dot2_bf16(fp4x2_to_bf16x2<0>(w), xv[4 * d + 0], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<1>(w), xv[4 * d + 1], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<2>(w), xv[4 * d + 2], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<3>(w), xv[4 * d + 3], acc);
  }
  return acc;
}

// ------------------------------------------------------------------------
// Routed gate/up: workgroup = (active expert a, tile of kRowsGU rows).
// CPL = code chunks per lane per row; MT = tokens held in registers at once.
template <int CPL, int MT>
__device__ void routed_gateup(const GemvLayer& L, int a, int tile) {
  if (a >= L.plan.n_active[0]) return;
  const int e = L.plan.active[a];
  const int p0 = L.plan.act_off[a];
  const int p1 = L.plan.act_off[a + 1];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int H = L.H, I = L.I;
  const int nch = H / 32;
  const size_t code_bytes = size_t(I) * H / 2;
  const size_t scale_bytes = size_t(I) * H / 32;
  const uint8_t* gc = L.experts + size_t(e) * L.stride;
  const uint8_t* gs = gc + code_bytes;
  const uint8_t* uc = gs + scale_bytes;
  const uint8_t* us = uc + code_bytes;

  for (int g0 = p0; g0 < p1; g0 += MT) {
    uint32_t xr[MT][CPL][16];
    int pr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const bool valid = g0 + t < p1;
      pr[t] = valid ? L.plan.pairs[g0 + t] : -1;
      const int tok = valid ? min(pr[t] / L.k, L.T - 1) : 0;
      const uint16_t* xrow = L.x + size_t(tok) * H;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + kWave * i;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 q = (valid && c < nch) ? ld16(xrow + c * 32 + v * 8) : u32x4{0, 0, 0, 0};
          xr[t][i][4 * v + 0] = q[0];
          xr[t][i][4 * v + 1] = q[1];
          xr[t][i][4 * v + 2] = q[2];
          xr[t][i][4 * v + 3] = q[3];
        }
      }
    }
#pragma unroll 2
    for (int q = 0; q < kRowsGU / kWaves; ++q) {
      const int r = tile * kRowsGU + wave + kWaves * q;
      const uint8_t* grow = gc + size_t(r) * (H / 2);
      const uint8_t* urow = uc + size_t(r) * (H / 2);
      u32x4 gw[CPL], uw[CPL];
      uint32_t gsb[CPL], usb[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + kWave * i;
        if (c < nch) {
          gw[i] = ld_nt(grow + c * 16);
          uw[i] = ld_nt(urow + c * 16);
          gsb[i] = gs[size_t(r) * nch + c];
          usb[i] = us[size_t(r) * nch + c];
        } else {
          gw[i] = uw[i] = u32x4{0, 0, 0, 0};
          gsb[i] = usb[i] = 127;
        }
      }
      float ag[MT], au[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) ag[t] = au[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const float sg = e8m0_to_f32(gsb[i]);
        const float su = e8m0_to_f32(usb[i]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          ag[t] = fmaf(block_dot_bf16(gw[i], xr[t][i], 0.0f), sg, ag[t]);
          au[t] = fmaf(block_dot_bf16(uw[i], xr[t][i], 0.0f), su, au[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float g = wave_sum(ag[t]);
        const float u = wave_sum(au[t]);
        if (lane == 0 && pr[t] >= 0) L.h[size_t(pr[t]) * I + r] = silu(g) * u;
      }
    }
  }
}

// Shared gate/up (bf16 weights): workgroup = (shared expert s, tile of
// kRowsGUS rows, one per wave); all T tokens, MT at a time, staged in LDS.
// CPLS = 16-byte chunks (8 bf16) per lane per row, consumed 4 at a time.
template <int CPLS, int MT>
__device__ void shared_gateup(const GemvLayer& L, int s, int tile, u32x4* xs) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int H = L.H, I = L.I;
  const int nch = H / 8;
  const uint16_t* G = L.sgate + size_t(s) * I * H;
  const uint16_t* U = L.sup + size_t(s) * I * H;
  const int r = tile * kRowsGUS + wave;
  const uint16_t* grow = G + size_t(r) * H;
  const uint16_t* urow = U + size_t(r) * H;
  for (int t0 = 0; t0 < L.T; t0 += MT) {
    const int nt = min(MT, L.T - t0);
    __syncthreads();
    const u32x4* src = reinterpret_cast<const u32x4*>(L.x + size_t(t0) * H);
    for (int i = threadIdx.x; i < nt * nch; i += kThreads) xs[i] = src[i];
    __syncthreads();
    float ag[MT], au[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ag[t] = au[t] = 0.0f;
#pragma unroll
    for (int i0 = 0; i0 < CPLS; i0 += 4) {
      u32x4 gw[4], uw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = lane + kWave * (i0 + i);
        gw[i] = c < nch ? ld_nt(grow + c * 8) : u32x4{0, 0, 0, 0};
        uw[i] = c < nch ? ld_nt(urow + c * 8) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = lane + kWave * (i0 + i);
        if (c < nch) {
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < nt) {
              const u32x4 xv = xs[t * nch + c];
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                ag[t] = dot2_bf16(gw[i][d], xv[d], ag[t]);
                au[t] = dot2_bf16(uw[i][d], xv[d], au[t]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float g = wave_sum(ag[t]);
      const float u = wave_sum(au[t]);
      if (lane == 0 && t < nt) L.hs[(size_t(s) * L.T + t0 + t) * I + r] = silu(g) * u;
    }
  }
}

// Grid: [shared tiles (S * I / kRowsGUS)] then [max_active * I / kRowsGU].
template <int CPL, int MT>
__global__ __launch_bounds__(kThreads) void gateup_kernel(GemvLayer L) {
  __shared__ u32x4 xs[kSharedTokens * 1024];  // kSharedTokens rows of H <= 8192 bf16
  const int shared_wgs = L.S * (L.I / kRowsGUS);
  const int b = blockIdx.x;
  if (b < shared_wgs) {
    const int tiles = L.I / kRowsGUS;
    shared_gateup<4 * CPL, kSharedTokens>(L, b / tiles, b % tiles, xs);
  } else {
    const int tiles = L.I / kRowsGU;
    const int r = b - shared_wgs;
    routed_gateup<CPL, MT>(L, r / tiles, r % tiles);
  }
}

// ------------------------------------------------------------------------
// Routed down: workgroup = (active expert a, tile of kRowsD output rows).
// part[pair][n] = sum_k Wd[n][k] h[pair][k]  (unweighted).
template <int CPL, int MT>
__device__ void routed_down(const GemvLayer& L, int a, int tile) {
  if (a >= L.plan.n_active[0]) return;
  const int e = L.plan.active[a];
  const int p0 = L.plan.act_off[a];
  const int p1 = L.plan.act_off[a + 1];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int H = L.H, I = L.I;
  const int nch = I / 32;
  const size_t gu_bytes = 2 * (size_t(I) * H / 2 + size_t(I) * H / 32);
  const uint8_t* dc = L.experts + size_t(e) * L.stride + gu_bytes;
  const uint8_t* ds = dc + size_t(H) * I / 2;

  for (int g0 = p0; g0 < p1; g0 += MT) {
    float hr[MT][CPL][32];
    int pr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const bool valid = g0 + t < p1;
      pr[t] = valid ? L.plan.pairs[g0 + t] : -1;
      const float* hrow = L.h + size_t(valid ? pr[t] : 0) * I;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + kWave * i;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const u32x4 q = (valid && c < nch) ? ld16(hrow + c * 32 + v * 4) : u32x4{0, 0, 0, 0};
          hr[t][i][4 * v + 0] = __uint_as_float(q[0]);
          hr[t][i][4 * v + 1] = __uint_as_float(q[1]);
          hr[t][i][4 * v + 2] = __uint_as_float(q[2]);
          hr[t][i][4 * v + 3] = __uint_as_float(q[3]);
        }
      }
    }
#pragma unroll 2
    for (int q = 0; q < kRowsD / kWaves; ++q) {
      const int n = tile * kRowsD + wave + kWaves * q;
      const uint8_t* row = dc + size_t(n) * (I / 2);
      u32x4 w[CPL];
      uint32_t sb[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + kWave * i;
        if (c < nch) {
          w[i] = ld_nt(row + c * 16);
          sb[i] = ds[size_t(n) * nch + c];
        } else {
          w[i] = u32x4{0, 0, 0, 0};
          sb[i] = 127;
        }
      }
      float acc[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const float sc = e8m0_to_f32(sb[i]);
        float blk[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) blk[t] = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t cw = w[i][d];
          const f32x2_t v0 = fp4x2_to_f32x2<0>(cw);
          const f32x2_t v1 = fp4x2_to_f32x2<1>(cw);
          const f32x2_t v2 = fp4x2_to_f32x2<2>(cw);
          const f32x2_t v3 = fp4x2_to_f32x2<3>(cw);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const float* hv = &hr[t][i][8 * d];
            float b = blk[t];
            b = fmaf(v0[0], hv[0], b);
            b = fmaf(v0[1], hv[1], b);
            b = fmaf(v1[0], hv[2], b);
            b = fmaf(v1[1], hv[3], b);
            b = fmaf(v2[0], hv[4], b);
            b = fmaf(v2[1], hv[5], b);
            b = fmaf(v3[0], hv[6], b);
            b = fmaf(v3[1], hv[7], b);
            blk[t] = b;
          }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = fmaf(blk[t], sc, acc[t]);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float y = wave_sum(acc[t]);
        if (lane == 0 && pr[t] >= 0) L.part[size_t(pr[t]) * H + n] = y;
      }
    }
  }
}

// Shared down (bf16): workgroup = tile of kRowsDS output rows, all shared
// experts and all tokens; ysh[t][n] = sum_s sum_k Wd_s[n][k] hs[s][t][k].
template <int CPLS, int MT>
__device__ void shared_down(const GemvLayer& L, int tile) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int H = L.H, I = L.I;
  const int nch = I / 8;
  constexpr int NQ = kRowsDS / kWaves;
  for (int t0 = 0; t0 < L.T; t0 += MT) {
    float acc[NQ][MT];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[q][t] = 0.0f;
    for (int s = 0; s < L.S; ++s) {
      float hr[MT][CPLS][8];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const bool valid = t0 + t < L.T;
        const float* hrow = L.hs + (size_t(s) * L.T + (valid ? t0 + t : 0)) * I;
#pragma unroll
        for (int i = 0; i < CPLS; ++i) {
          const int c = lane + kWave * i;
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const u32x4 q = (valid && c < nch) ? ld16(hrow + c * 8 + v * 4) : u32x4{0, 0, 0, 0};
            hr[t][i][4 * v + 0] = __uint_as_float(q[0]);
            hr[t][i][4 * v + 1] = __uint_as_float(q[1]);
            hr[t][i][4 * v + 2] = __uint_as_float(q[2]);
            hr[t][i][4 * v + 3] = __uint_as_float(q[3]);
          }
        }
      }
      const uint16_t* D = L.sdown + size_t(s) * H * I;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int n = tile * kRowsDS + wave + kWaves * q;
        u32x4 w[CPLS];
#pragma unroll
        for (int i = 0; i < CPLS; ++i) {
          const int c = lane + kWave * i;
          w[i] = c < nch ? ld_nt(D + size_t(n) * I + c * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < CPLS; ++i)
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            float b = acc[q][t];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              b = fmaf(bf16_lo(w[i][d]), hr[t][i][2 * d], b);
              b = fmaf(bf16_hi(w[i][d]), hr[t][i][2 * d + 1], b);
            }
            acc[q][t] = b;
          }
      }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int n = tile * kRowsDS + wave + kWaves * q;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float y = wave_sum(acc[q][t]);
        if (lane == 0 && t0 + t < L.T) L.ysh[size_t(t0 + t) * H + n] = y;
      }
    }
  }
}

// Grid: [shared tiles (H / kRowsDS, when S > 0)] then [max_active * H / kRowsD].
template <int CPL, int MT>
__global__ __launch_bounds__(kThreads) void down_kernel(GemvLayer L) {
  const int shared_wgs = L.S > 0 ? L.H / kRowsDS : 0;
  const int b = blockIdx.x;
  if (b < shared_wgs) {
    shared_down<4 * CPL, MT>(L, b);
  } else {
    const int tiles = L.H / kRowsD;
    const int r = b - shared_wgs;
    routed_down<CPL, MT>(L, r / tiles, r % tiles);
  }
}

// ------------------------------------------------------------------------
// y[t][n] = bf16( sum_j w[t][j] part[t*k+j][n] + ysh[t][n] + residual[t][n] ),
// eight outputs per thread, summed in that order.
__global__ __launch_bounds__(256) void combine_kernel(GemvLayer L, const float* __restrict__ w,
                                                      const uint16_t* __restrict__ residual,
                                                      uint16_t* __restrict__ y) {
  const int H = L.H;
  const int nch = H / 8;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= size_t(L.T) * nch) return;
  const int t = int(idx / nch);
  const int c = int(idx % nch);
  float acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = 0.0f;
  for (int j = 0; j < L.k; ++j) {
    const size_t p = size_t(t) * L.k + j;
    const float wj = w[p];
    const float* src = L.part + p * H + c * 8;
    const u32x4 a = ld16(src);
    const u32x4 b = ld16(src + 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[v] = fmaf(wj, __uint_as_float(a[v]), acc[v]);
      acc[4 + v] = fmaf(wj, __uint_as_float(b[v]), acc[4 + v]);
    }
  }
  if (L.S > 0) {
    const float* src = L.ysh + size_t(t) * H + c * 8;
    const u32x4 a = ld16(src);
    const u32x4 b = ld16(src + 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[v] += __uint_as_float(a[v]);
      acc[4 + v] += __uint_as_float(b[v]);
    }
  }
  if (residual != nullptr) {
    const u32x4 r = ld16(residual + size_t(t) * H + c * 8);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[2 * v] += bf16_lo(r[v]);
      acc[2 * v + 1] += bf16_hi(r[v]);
    }
  }
  u32x4 o;
#pragma unroll
  for (int v = 0; v < 4; ++v)
    o[v] = uint32_t(f32_to_bf16(acc[2 * v])) | (uint32_t(f32_to_bf16(acc[2 * v + 1])) << 16);
  *reinterpret_cast<u32x4*>(y + size_t(t) * H + c * 8) = o;
}

int cpl_for(int chunks) { return chunks <= 64 ? 1 : (chunks <= 128 ? 2 : 4); }

}  // namespace

using GemvKernel = void (*)(GemvLayer);

template <template <int, int> class Pick>
GemvKernel pick(int cpl, int mt) {
  if (cpl == 1) return mt == 1 ? Pick<1, 1>::fn : Pick<1, 2>::fn;
  if (cpl == 2) return mt == 1 ? Pick<2, 1>::fn : Pick<2, 2>::fn;
  return mt == 1 ? Pick<4, 1>::fn : Pick<4, 2>::fn;
}

template <int CPL, int MT>
struct PickGateUp {
  static constexpr GemvKernel fn = gateup_kernel<CPL, MT>;
};

template <int CPL, int MT>
struct PickDown {
  static constexpr GemvKernel fn = down_kernel<CPL, MT>;
};

hipError_t launch_gateup(const GemvLayer& L, hipStream_t stream) {
  const int cpl = cpl_for(L.H / 32);
  const int mt = L.T > 1 ? 2 : 1;
  const int wgs = L.S * (L.I / kRowsGUS) + L.max_active * (L.I / kRowsGU);
  hipLaunchKernelGGL(pick<PickGateUp>(cpl, mt), dim3(wgs), dim3(kThreads), 0, stream, L);
  return hipGetLastError();
}

hipError_t launch_down(const GemvLayer& L, hipStream_t stream) {
  const int cpl = cpl_for(L.I / 32);
  const int mt = L.T > 1 ? 2 : 1;
  const int wgs = (L.S > 0 ? L.H / kRowsDS : 0) + L.max_active * (L.H / kRowsD);
  hipLaunchKernelGGL(pick<PickDown>(cpl, mt), dim3(wgs), dim3(kThreads), 0, stream, L);
  return hipGetLastError();
}

hipError_t launch_combine(const GemvLayer& L, const float* w,
                          const uint16_t* residual, uint16_t* y, hipStream_t stream) {
  const size_t n = size_t(L.T) * (L.H / 8);
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, L, w,
                     residual, y);
  return hipGetLastError();
}

}  // namespace moe
