// The step's first launch: the tile schedule and the fused prologue in one
// kernel.  They are independent (the schedule reads only the lengths), so
// block 0 computes the schedule while the other blocks run the prologue rows,
// saving a launch and letting the two overlap.
//
// Launch: 1 + ceil(batch * Tq * runs / 16) blocks of 1024 threads, one wave per
// run of consecutive rows of a token (rows = Hq + 2 Hkv; runs per token from
// prologue_runs_per_token, one row per run at decode sizes);
// dynamic LDS of batch + 1 ints (the schedule's prefix sums).

#include "launch.h"
#include "plan.h"
#include "prologue.h"

namespace lbsr {

template <bool kFp8, bool kOneRow>
__global__ __launch_bounds__(kPlanThreads) void plan_prologue_kernel(
    const int32_t* __restrict__ seq_lens, SchedParams sp, PlanPtrs plan, Geometry geo, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ positions,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const int32_t* __restrict__ block_table, void* __restrict__ k_cache,
    void* __restrict__ v_cache, uint16_t* __restrict__ q_out, RopeFreqs freqs, double eps,
    int norm_first, double k_scale, double v_scale, int runs) {
  extern __shared__ int s_cu[];
  if (blockIdx.x == 0) {
    plan_body(seq_lens, geo.batch, geo.max_blocks, sp, plan, s_cu);
    return;
  }
  const int rows = geo.num_q_heads + 2 * geo.num_kv_heads;
  const int wv = (blockIdx.x - 1) * (kPlanThreads / kWave) + (threadIdx.x >> 6);
  if (wv >= geo.batch * geo.tokens * runs) return;
  const int tok = wv / runs, i = wv - tok * runs;
  // Block 0 clears the error word concurrently, so the prologue rows do not
  // touch it: each token's status is stored (overwritten every step) and the
  // merge kernel, which runs after both, folds it into the error word.
  const int rb = kOneRow ? i : prologue_run_begin(i, runs, rows);
  const int re = kOneRow ? i + 1 : prologue_run_begin(i + 1, runs, rows);
  prologue_rows<kFp8, kOneRow>(tok, tok / geo.tokens, rb, re, geo, q, k, v, positions, wq, wk,
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
  const int runs = prologue_runs_per_token(geo.batch * geo.tokens, rows);
  const int blocks =
      1 + (geo.batch * geo.tokens * runs + kPlanThreads / kWave - 1) / (kPlanThreads / kWave);
  const size_t lds = sizeof(int) * (size_t)(geo.batch + 1);
  auto* qq = (const uint16_t*)q;
  auto* kk = (const uint16_t*)k;
  auto* vv = (const uint16_t*)v;
  auto kernel = fp8 ? (runs == rows ? plan_prologue_kernel<true, true>
                                   : plan_prologue_kernel<true, false>)
                   : (runs == rows ? plan_prologue_kernel<false, true>
                                   : plan_prologue_kernel<false, false>);
  kernel<<<blocks, kPlanThreads, lds, stream>>>(
      seq_lens, sp, plan, geo, qq, kk, vv, positions, (const uint16_t*)wq, (const uint16_t*)wk,
      block_table, k_cache, v_cache, (uint16_t*)q_out, freqs, eps, norm_first, k_scale, v_scale,
      runs);
  return hipGetLastError();
}

}  // namespace lbsr
