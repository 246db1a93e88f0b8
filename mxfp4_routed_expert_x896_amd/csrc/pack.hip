// Weight repacking into the MFMA-tiled layout the expert kernels stream.
//
// MXFP4 matrix, R rows (multiple of 16) x K columns (multiple of 32),
// nb = K / 32 blocks per row, nkb = ceil(nb / 4), nkb4 = nkb rounded up to
// a multiple of 4:
//   codes: tile (rg, kb), rg < R / 16, kb < nkb, is 1024 contiguous bytes at
//     (rg * nkb + kb) * 1024; bytes [16 l, 16 l + 16), l = 16 g + c, are the
//     codes of block 4 kb + g of row 16 rg + c (zeros past the last block);
//   scales: after the codes, byte ((rg * nkb4 / 4 + kb / 4) * 64 + l) * 4 +
//     kb % 4 is that block's E8M0 scale (127 past the last block).
// One wave64 load of a tile is 1 KiB of contiguous codes whose lane l holds
// exactly the 32 elements the MFMA A operand of lane l needs; a lane's
// scales for four consecutive tiles (a super-step) are one aligned dword,
// and the 64 lanes' dwords of a super-step are 256 contiguous bytes.
//
// bf16 matrix, R rows (multiple of 16) x K columns (multiple of 32):
//   tile (rg, u) for u < K / 32 is 1024 contiguous bytes; lane l = 16 g + c
//   holds elements 32 u + 8 g .. 32 u + 8 g + 7 of row 16 rg + c.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// One thread per (tile, lane): copies 16 code bytes and one scale byte.
__global__ __launch_bounds__(256) void pack_mxfp4_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         int R, int K, uint8_t* __restrict__ dst) {
  const int nb = K / 32;
  const int nkb = (nb + 3) / 4;
  const size_t n = size_t(R / 16) * nkb * 64;
  const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int l = int(i % 64);
  const size_t tile = i / 64;
  const int kb = int(tile % nkb);
  const int rg = int(tile / nkb);
  const int g = l / 16, c = l % 16;
  const int row = rg * 16 + c;
  const int bi = 4 * kb + g;
  const int nkb4 = (nkb + 3) / 4 * 4;
  u32x4 v = u32x4{0, 0, 0, 0};
  uint8_t s = 127;
  if (bi < nb) {
    v = *reinterpret_cast<const u32x4*>(codes + size_t(row) * (K / 2) + size_t(bi) * 16);
    s = scales[size_t(row) * nb + bi];
  }
  *reinterpret_cast<u32x4*>(dst + tile * 1024 + 16 * l) = v;
  uint8_t* sc = dst + size_t(R / 16) * nkb * 1024;
  const size_t row_sc = size_t(rg) * (nkb4 / 4) * 256 + 4 * l;  // lane l's dwords, 256 apart
  sc[row_sc + size_t(kb / 4) * 256 + kb % 4] = s;
  if (kb == nkb - 1)  // padding scales of the row group's last dword
    for (int k2 = nkb; k2 < nkb4; ++k2) sc[row_sc + size_t(k2 / 4) * 256 + k2 % 4] = 127;
}

__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t* __restrict__ src, int R,
                                                        int K, uint16_t* __restrict__ dst) {
  const int nu = K / 32;
  const size_t n = size_t(R / 16) * nu * 64;
  const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int l = int(i % 64);
  const size_t tile = i / 64;
  const int u = int(tile % nu);
  const int rg = int(tile / nu);
  const int g = l / 16, c = l % 16;
  const u32x4 v =
      *reinterpret_cast<const u32x4*>(src + size_t(rg * 16 + c) * K + size_t(u) * 32 + 8 * g);
  *reinterpret_cast<u32x4*>(dst + tile * 512 + 8 * l) = v;
}

}  // namespace

size_t packed_mxfp4_bytes(int R, int K) { return PackedMx(R, K).bytes; }

size_t packed_record_bytes(int H, int I) {
  return 2 * packed_mxfp4_bytes(I, H) + packed_mxfp4_bytes(H, I);
}

hipError_t launch_pack_record(const uint8_t* src, int H, int I, uint8_t* dst,
                              hipStream_t stream) {
  const size_t gu_codes = size_t(I) * H / 2, gu_scales = size_t(I) * H / 32;
  const uint8_t* m_codes[3] = {src, src + gu_codes + gu_scales, src + 2 * (gu_codes + gu_scales)};
  const int rows[3] = {I, I, H};
  const int cols[3] = {H, H, I};
  uint8_t* d = dst;
  for (int m = 0; m < 3; ++m) {
    const uint8_t* sc = m_codes[m] + size_t(rows[m]) * cols[m] / 2;
    const size_t n = size_t(rows[m] / 16) * ((cols[m] / 32 + 3) / 4) * 64;
    hipLaunchKernelGGL(pack_mxfp4_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream,
                       m_codes[m], sc, rows[m], cols[m], d);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    d += packed_mxfp4_bytes(rows[m], cols[m]);
  }
  return hipSuccess;
}

hipError_t launch_pack_bf16(const uint16_t* src, int R, int K, uint16_t* dst, hipStream_t stream) {
  const size_t n = size_t(R / 16) * (K / 32) * 64;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, src,
                     R, K, dst);
  return hipGetLastError();
}

}  // namespace moe
