// Row-scaled int8 -> fp32 expansion of a dense weight matrix.
//
// Deltafin README, Techniques / Compute: the dense weights are stored as
// int8 with one scale per row, and one fused kernel converts, multiplies by
// the row's scale and copies into the fp32 buffer (bit-exact against the
// unfused path).  out[r][c] = float(q[r][c]) * scale[r]: the conversion is
// exact and the product is the one rounding.
//
// Pure streaming: 1 byte read and 4 bytes written per element (plus one
// scale per row), so the roof is HBM bandwidth.  A workgroup of two waves
// takes 1024 elements of one row; in each of 2 steps a wave reads 256
// contiguous bytes (one dword per lane) and writes 1 KiB contiguous (16
// bytes per lane), both loads issued before the first store.  Stores are
// non-temporal: the output is not read again by this kernel and should not
// displace the L2.  Measured on 32768 x 7168: small workgroups with few
// steps stream best (128 x 2 steps: 82% of the HBM peak; 256 x 4: 71%;
// 256 x 7 or persistent grids: 64-67%).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kDqThreads = 128;
constexpr int kDqSteps = 2;
constexpr int kDqChunk = kDqThreads * 4 * kDqSteps;  // elements of a row per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 expand(uint32_t v, float s) {
  f32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = float(int8_t(v >> (8 * i))) * s;
  return o;
}

__global__ __launch_bounds__(kDqThreads) void int8_row_dequant_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ scale, int64_t cols,
    uint32_t chunks_per_row, float* __restrict__ out) {
  const uint32_t b = blockIdx.x;
  const uint32_t r = b / chunks_per_row;
  const int64_t start = int64_t(b - r * chunks_per_row) * kDqChunk;
  const int64_t c0 = start + 4 * threadIdx.x;
  const float s = scale[r];
  const int8_t* qrow = q + int64_t(r) * cols;
  float* orow = out + int64_t(r) * cols;
  uint32_t v[kDqSteps];
  if (start + kDqChunk <= cols) {
    // whole chunk inside the row (the workgroup agrees): no per-lane
    // conditions, so the loads are waited for once and the stores issue
    // back to back
#pragma unroll
    for (int j = 0; j < kDqSteps; ++j)
      v[j] = *reinterpret_cast<const uint32_t*>(qrow + c0 + j * kDqThreads * 4);
    f32x4 o[kDqSteps];
#pragma unroll
    for (int j = 0; j < kDqSteps; ++j) o[j] = expand(v[j], s);
#pragma unroll
    for (int j = 0; j < kDqSteps; ++j)
      __builtin_nontemporal_store(o[j], reinterpret_cast<f32x4*>(orow + c0 + j * kDqThreads * 4));
    return;
  }
  // the row's last, partial chunk (cols is a multiple of 4, so a lane's
  // four elements are all inside or all outside)
#pragma unroll
  for (int j = 0; j < kDqSteps; ++j) {
    const int64_t c = c0 + j * kDqThreads * 4;
    v[j] = *reinterpret_cast<const uint32_t*>(qrow + min(c, cols - 4));
  }
#pragma unroll
  for (int j = 0; j < kDqSteps; ++j) {
    const int64_t c = c0 + j * kDqThreads * 4;
    if (c < cols) __builtin_nontemporal_store(expand(v[j], s), reinterpret_cast<f32x4*>(orow + c));
  }
}

}  // namespace

int64_t int8_dequant_blocks(int64_t rows, int64_t cols) {
  return rows * ((cols + kDqChunk - 1) / kDqChunk);
}

hipError_t launch_int8_row_dequant(const int8_t* q, const float* scale, int64_t rows, int64_t cols,
                                   float* out, hipStream_t stream) {
  const uint32_t cpr = uint32_t((cols + kDqChunk - 1) / kDqChunk);
  launch_timed(next_launch_events(), int8_row_dequant_kernel, dim3(uint32_t(rows * cpr)),
               dim3(kDqThreads), 0u, stream, q, scale, cols, cpr, out);
  return hipGetLastError();
}

}  // namespace moe
