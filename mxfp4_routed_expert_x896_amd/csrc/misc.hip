// RMSNorm for stacked layers, the MXFP8 activation quantiser, and the
// dequantised-weight export used to check the MXFP4 decode bit for bit.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// ------------------------------------------------------------- RMSNorm ----
// One workgroup of 256 threads per token; H <= 8192 (at most 4 chunks of 8
// bf16 per thread).  out = bf16(x * (mean(x^2) + eps)^-1/2 * gamma).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ gamma,
                                                      float eps, int H, uint16_t* out) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const int nch = H / 8;
  const uint16_t* row = x + size_t(t) * H;
  u32x4 v[4];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + 256 * i;
    v[i] = c < nch ? *reinterpret_cast<const u32x4*>(row + c * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float a = bf16_lo(v[i][d]);
      const float b = bf16_hi(v[i][d]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  ss = wave_sum(ss);
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float r = 1.0f / sqrtf(tot / float(H) + eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nch) {
      const u32x4 g = *reinterpret_cast<const u32x4*>(gamma + c * 8);
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float lo = bf16_lo(v[i][d]) * r * bf16_lo(g[d]);
        const float hi = bf16_hi(v[i][d]) * r * bf16_hi(g[d]);
        o[d] = uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
      }
      *reinterpret_cast<u32x4*>(out + size_t(t) * H + c * 8) = o;
    }
  }
}

// ---------------------------------------------------- dequant export -----
// One thread per (packed tile, lane): the lane's 16 code bytes are decoded by
// the same scaled convert the expert kernels use (fp4x8_scaled), widened to
// fp32 and written at their canonical place out[row][k].
__global__ __launch_bounds__(256) void dequant_export_kernel(const uint8_t* __restrict__ mat,
                                                             int rows, int cols,
                                                             float* __restrict__ out) {
  const PackedMx pm(rows, cols);
  const size_t n = size_t(rows / 16) * pm.nkb * 64;
  const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int l = int(i % 64);
  const size_t tile = i / 64;
  const int kb = int(tile % pm.nkb);
  const int rg = int(tile / pm.nkb);
  const int bi = 4 * kb + l / 16;
  if (bi >= pm.nb) return;
  const int row = rg * 16 + l % 16;
  const u32x4 codes = *reinterpret_cast<const u32x4*>(mat + tile * 1024 + 16 * l);
  const float sc = e8m0_to_f32(mat[pm.scale_dword(rg, kb / 4, l) + kb % 4]);
  float* o = out + size_t(row) * cols + size_t(bi) * 32;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x4 v = fp4x8_scaled(codes[d], sc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[8 * d + 2 * q] = bf16_lo(v[q]);
      o[8 * d + 2 * q + 1] = bf16_hi(v[q]);
    }
  }
}

// -------------------------------------------------------------- MXFP8 -----

// One thread per 32-element block: E = clamp(floor(log2 amax) - 8, -127,
// 127) (-127 for an all-zero block), codes = E4M3(v / 2^E).
__global__ __launch_bounds__(256) void mxfp8_quant_kernel(const uint16_t* __restrict__ x,
                                                          size_t n_blocks,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const size_t b = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= n_blocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + b * 32);
  u32x4 v[4];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = src[i];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i][d])), fabsf(bf16_hi(v[i][d]))));
  }
  const int E = mxfp8_block_exp(amax);
  uint32_t words[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // elements 8i+2d and 8i+2d+1 -> bytes 8i+2d, 8i+2d+1 of the block
      const uint32_t c0 = e4m3_rne_sat(__builtin_ldexpf(bf16_lo(v[i][d]), -E));
      const uint32_t c1 = e4m3_rne_sat(__builtin_ldexpf(bf16_hi(v[i][d]), -E));
      const uint32_t half = c0 | (c1 << 8);
      if (d % 2 == 0)
        words[2 * i + d / 2] = half;
      else
        words[2 * i + d / 2] |= half << 16;
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(codes + b * 32);
  dst[0] = u32x4{words[0], words[1], words[2], words[3]};
  dst[1] = u32x4{words[4], words[5], words[6], words[7]};
  scales[b] = uint8_t(E + 127);
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H,
                          uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, stream, x, gamma, eps, H, out);
  return hipGetLastError();
}

hipError_t launch_dequant_export(const uint8_t* record, int H, int I, int matrix, float* out,
                                 hipStream_t stream) {
  const uint8_t* mat = record + size_t(matrix) * packed_mxfp4_bytes(I, H);
  const int rows = matrix == 2 ? H : I;
  const int cols = matrix == 2 ? I : H;
  const size_t n = size_t(rows / 16) * PackedMx(rows, cols).nkb * 64;
  hipLaunchKernelGGL(dequant_export_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream,
                     mat, rows, cols, out);
  return hipGetLastError();
}

hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int K, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream) {
  const size_t nb = size_t(rows) * (K / 32);
  hipLaunchKernelGGL(mxfp8_quant_kernel, dim3(unsigned((nb + 255) / 256)), dim3(256), 0, stream,
                     x, nb, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
