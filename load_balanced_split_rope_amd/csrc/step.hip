// The step's first launch: the tile schedule and the fused prologue in one
// kernel.  They are independent (the schedule reads only the lengths), so
// block 0 computes the schedule while the other blocks run the prologue rows,
// saving a launch and letting the two overlap.
//
// Launch: 1 + ceil(batch * Tq * rows / 16) blocks of 1024 threads, rows = Hq + 2 Hkv;
// dynamic LDS of batch + 1 ints (the schedule's prefix sums).

#include "launch.h"
#include "plan.h"
#include "prologue.h"

namespace lbsr {

template <bool kFp8>
__global__ __launch_bounds__(kPlanThreads) void plan_prologue_kernel(
    const int32_t* __restrict__ seq_lens, SchedParams sp, PlanPtrs plan, Geometry geo, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ positions,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const int32_t* __restrict__ block_table, void* __restrict__ k_cache,
    void* __restrict__ v_cache, uint16_t* __restrict__ q_out, RopeFreqs freqs, double eps,
    int norm_first, double k_scale, double v_scale) {
  extern __shared__ int s_cu[];
  if (blockIdx.x == 0) {
    plan_body(seq_lens, geo.batch, geo.max_blocks, sp, plan, s_cu);
    return;
  }
  const int rows = geo.num_q_heads + 2 * geo.num_kv_heads;
  const int r = (blockIdx.x - 1) * (kPlanThreads / kWave) + (threadIdx.x >> 6);
  if (r >= geo.batch * geo.tokens * rows) return;
  const int tok = r / rows;
  // Block 0 clears the error word concurrently, so the prologue rows do not
  // touch it: each token's status is stored (overwritten every step) and the
  // merge kernel, which runs after both, folds it into the error word.
  prologue_row<kFp8>(tok, tok / geo.tokens, r - tok * rows, geo, q, k, v, positions, wq, wk,
                     block_table, k_cache, v_cache, q_out, nullptr, plan.token_status, freqs,
                     eps, norm_first, k_scale, v_scale);
}

hipError_t launch_plan_prologue(const int32_t* seq_lens, const SchedParams& sp,
                                const PlanPtrs& plan, const Geometry& geo,
                                bool fp8, const void* q, const void* k, const void* v,
                                const int32_t* positions, const void* wq, const void* wk,
                                const int32_t* block_table, void* k_cache, void* v_cache,
                                void* q_out, const RopeFreqs& freqs, double eps, int norm_first,
                                double k_scale, double v_scale, hipStream_t stream) {
  const int rows = geo.num_q_heads + 2 * geo.num_kv_heads;
  const int blocks =
      1 + (geo.batch * geo.tokens * rows + kPlanThreads / kWave - 1) / (kPlanThreads / kWave);
  const size_t lds = sizeof(int) * (size_t)(geo.batch + 1);
  auto* qq = (const uint16_t*)q;
  auto* kk = (const uint16_t*)k;
  auto* vv = (const uint16_t*)v;
  if (fp8)
    plan_prologue_kernel<true><<<blocks, kPlanThreads, lds, stream>>>(
        seq_lens, sp, plan, geo, qq, kk, vv, positions,
        (const uint16_t*)wq, (const uint16_t*)wk, block_table, k_cache, v_cache,
        (uint16_t*)q_out, freqs, eps, norm_first, k_scale, v_scale);
  else
    plan_prologue_kernel<false><<<blocks, kPlanThreads, lds, stream>>>(
        seq_lens, sp, plan, geo, qq, kk, vv, positions,
        (const uint16_t*)wq, (const uint16_t*)wk, block_table, k_cache, v_cache,
        (uint16_t*)q_out, freqs, eps, norm_first, k_scale, v_scale);
  return hipGetLastError();
}

}  // namespace lbsr
