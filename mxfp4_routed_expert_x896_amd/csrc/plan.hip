// Stand-alone token -> expert plan for a routing supplied by the caller, so
// that every expert's weights stream from HBM once per call however many
// tokens chose it.
#include "kernels.hpp"
#include "plan.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ ids,
                                                            int n_pairs, int E, Plan plan,
                                                            int* zero, int n_zero) {
  build_plan(ids, n_pairs, E, plan, zero, n_zero);
}

}  // namespace

hipError_t launch_plan(const int32_t* ids, int n_pairs, int E, Plan plan, int* zero, int n_zero,
                       hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, ids, n_pairs, E, plan,
                     zero, n_zero);
  return hipGetLastError();
}

}  // namespace moe
