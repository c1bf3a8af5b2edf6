// The tile schedule as its own kernel (lbsr_plan); the code is in plan.h.

#include "launch.h"
#include "plan.h"

namespace lbsr {

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seq_lens,
                                                            int batch, int max_blocks,
                                                            int dynamic, int num_workers,
                                                            int splits, PlanPtrs plan) {
  extern __shared__ int s_cu[];
  plan_body(seq_lens, batch, max_blocks, dynamic, num_workers, splits, plan, s_cu);
}

hipError_t launch_plan(const int32_t* seq_lens, int batch, int max_blocks, bool dynamic,
                       int num_workers, int static_splits, const PlanPtrs& plan,
                       hipStream_t stream) {
  const size_t lds = sizeof(int) * (size_t)(batch + 1);
  plan_kernel<<<1, kPlanThreads, lds, stream>>>(seq_lens, batch, max_blocks, dynamic ? 1 : 0,
                                                 num_workers, static_splits, plan);
  return hipGetLastError();
}

}  // namespace lbsr
