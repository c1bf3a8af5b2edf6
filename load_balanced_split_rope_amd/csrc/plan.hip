// The tile schedule as its own kernel (lbsr_plan); the code is in plan.h.

#include "launch.h"
#include "plan.h"

namespace lbsr {

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seq_lens,
                                                            int batch, int max_blocks,
                                                            SchedParams sp, PlanPtrs plan) {
  extern __shared__ int s_cu[];
  plan_body(seq_lens, batch, max_blocks, sp, plan, s_cu);
}

hipError_t launch_plan(const int32_t* seq_lens, int batch, int max_blocks, const SchedParams& sp,
                       const PlanPtrs& plan, hipStream_t stream) {
  const size_t lds = sizeof(int) * (size_t)(batch + 1);
  plan_kernel<<<1, kPlanThreads, lds, stream>>>(seq_lens, batch, max_blocks, sp, plan);
  return hipGetLastError();
}

}  // namespace lbsr
