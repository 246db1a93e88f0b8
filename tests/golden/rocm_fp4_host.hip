// Prints ROCm's host-side decode of every packed FP4 (E2M1) byte:
// "<byte> <element 0> <element 1>".  Used as a library pin for the oracle's
// E2M1 table and nibble order; it runs on the CPU and launches no kernel.
#include <hip/hip_fp4.h>
#include <cstdio>

int main() {
  for (int b = 0; b < 256; ++b) {
    __hip_fp4x2_e2m1 v;
    v.__x = static_cast<__hip_fp4x2_storage_t>(b);
    float2 f = v;
    std::printf("%d %.9g %.9g\n", b, f.x, f.y);
  }
  return 0;
}
