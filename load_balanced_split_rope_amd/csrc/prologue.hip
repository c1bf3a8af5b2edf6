// The fused prologue as its own kernel (lbsr_rope_norm_kv_write).  The row
// code is in prologue.h.
//
// Launch: ceil(tokens * runs / 4) blocks of 256 threads, one wave per run of
// consecutive rows of a token; rows = Hq + 2 * Hkv, tokens = batch * Tq (or
// the packed count of a ragged batch, whose token -> sequence map is
// q_start), runs per token from prologue_runs_per_token.

#include "launch.h"
#include "prologue.h"

namespace lbsr {

template <bool kFp8, bool kOneRow>
__global__ __launch_bounds__(256) void prologue_kernel(
    Geometry geo, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ positions,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const int32_t* __restrict__ block_table, void* __restrict__ k_cache,
    void* __restrict__ v_cache, uint16_t* __restrict__ q_out, int32_t* __restrict__ error_word,
    RopeFreqs freqs, double eps, int norm_first, double k_scale, double v_scale, int runs,
    int num_tokens, const int32_t* __restrict__ q_start) {
  const int rows = geo.num_q_heads + 2 * geo.num_kv_heads;
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv >= num_tokens * runs) return;
  const int tok = wv / runs, i = wv - tok * runs;
  const int rb = kOneRow ? i : prologue_run_begin(i, runs, rows);
  const int re = kOneRow ? i + 1 : prologue_run_begin(i + 1, runs, rows);
  // the sequence only picks the block-table row of k/v rows
  const int seq = !q_start ? tok / geo.tokens
                           : (re > geo.num_q_heads ? seq_of_token(q_start, geo.batch, tok) : 0);
  prologue_rows<kFp8, kOneRow>(tok, seq, rb, re, geo, q, k, v, positions, wq, wk,
                               block_table, k_cache, v_cache, q_out, error_word, nullptr, freqs,
                               eps, norm_first, k_scale, v_scale);
}

hipError_t launch_prologue(const Geometry& geo, bool fp8, const void* q, const void* k,
                           const void* v, const int32_t* positions, const void* wq,
                           const void* wk, const int32_t* block_table, void* k_cache,
                           void* v_cache, void* q_out, int32_t* error_word, const RopeFreqs& freqs,
                           double eps, int norm_first, double k_scale, double v_scale,
                           int num_tokens, const int32_t* q_start, hipStream_t stream) {
  const int rows = geo.num_q_heads + 2 * geo.num_kv_heads;
  const int runs = prologue_runs_per_token(num_tokens, rows);
  const int grid = (num_tokens * runs + 3) / 4;
  auto kernel = fp8 ? (runs == rows ? prologue_kernel<true, true> : prologue_kernel<true, false>)
                   : (runs == rows ? prologue_kernel<false, true> : prologue_kernel<false, false>);
  kernel<<<grid, 256, 0, stream>>>(
      geo, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, positions,
      (const uint16_t*)wq, (const uint16_t*)wk, block_table, k_cache, v_cache, (uint16_t*)q_out,
      error_word, freqs, eps, norm_first, k_scale, v_scale, runs, num_tokens, q_start);
  return hipGetLastError();
}

}  // namespace lbsr
