// Matrix-core issue rate of the block-scaled 16x16x128 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4) for the operand formats the prefill
// path could use: FP4 x FP8 (what it uses: MXFP4 weights, MXFP8
// activations) and FP4 x FP4 (activations in MXFP4, a choice the Deltafin
// explainer, section 2.1, leaves open next to the MXFP8 activations of
// training), with FP8 x FP8 for reference.  Each wave keeps eight
// independent accumulators and issues `iters` rounds of eight MFMAs on
// register operands (no memory traffic inside the loop), so the launch's
// duration measures the instruction rate alone.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kRateAcc = 8;

template <int AF, int BF>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int64_t iters, float* out) {
  const int lane = threadIdx.x % kWave;
  // finite operand bytes (any E2M1 nibble is finite; E4M3 avoids 0x7F/0xFF)
  const int v = 0x11223344 ^ (lane * 0x01010101);
  const i32x8 a = {v & 0x6E6E6E6E, v >> 1 & 0x6E6E6E6E, v ^ 0x24242424, v & 0x3C3C3C3C,
                   v & 0x5A5A5A5A, v & 0x2D2D2D2D, v & 0x4B4B4B4B, v & 0x36363636};
  const i32x8 b = {v & 0x3C3C3C3C, v & 0x5A5A5A5A, v & 0x6E6E6E6E, v & 0x2D2D2D2D,
                   v & 0x4B4B4B4B, v & 0x36363636, v & 0x24242424, v & 0x1E1E1E1E};
  f32x4 acc[kRateAcc];
#pragma unroll
  for (int i = 0; i < kRateAcc; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kRateAcc; ++i)
      acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i], AF, BF, 0, 127, 0,
                                                                127);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kRateAcc; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  if (lane == 0) out[blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave] = s;
}

}  // namespace

hipError_t launch_mfma_rate(int a_fmt, int b_fmt, int64_t iters, int blocks, float* out,
                            hipStream_t stream) {
  const LaunchEvents ev = next_launch_events();
  const dim3 grid(blocks), block(256);
  if (a_fmt == 4 && b_fmt == 4)
    launch_timed(ev, mfma_rate_kernel<4, 4>, grid, block, 0, stream, iters, out);
  else if (a_fmt == 4 && b_fmt == 0)
    launch_timed(ev, mfma_rate_kernel<4, 0>, grid, block, 0, stream, iters, out);
  else if (a_fmt == 0 && b_fmt == 0)
    launch_timed(ev, mfma_rate_kernel<0, 0>, grid, block, 0, stream, iters, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
