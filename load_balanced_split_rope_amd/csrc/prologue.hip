// The fused prologue as its own kernel (lbsr_rope_norm_kv_write).  The row
// code is in prologue.h.
//
// Launch: ceil(tokens * rows / 4) blocks of 256 threads, one wave per row;
// rows = Hq + 2 * Hkv, tokens = batch * Tq.

#include "launch.h"
#include "prologue.h"

namespace lbsr {

template <bool kFp8>
__global__ __launch_bounds__(256) void prologue_kernel(
    Geometry geo, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ positions,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const int32_t* __restrict__ block_table, void* __restrict__ k_cache,
    void* __restrict__ v_cache, uint16_t* __restrict__ q_out, int32_t* __restrict__ error_word,
    RopeFreqs freqs, double eps, int norm_first, double k_scale, double v_scale) {
  const int rows = geo.num_q_heads + 2 * geo.num_kv_heads;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= geo.batch * geo.tokens * rows) return;
  const int tok = r / rows;
  prologue_row<kFp8>(tok, tok / geo.tokens, r - tok * rows, geo, q, k, v, positions, wq, wk,
                     block_table, k_cache, v_cache, q_out, error_word, nullptr, freqs, eps,
                     norm_first, k_scale, v_scale);
}

hipError_t launch_prologue(const Geometry& geo, bool fp8, const void* q, const void* k,
                           const void* v, const int32_t* positions, const void* wq,
                           const void* wk, const int32_t* block_table, void* k_cache,
                           void* v_cache, void* q_out, int32_t* error_word, const RopeFreqs& freqs,
                           double eps, int norm_first, double k_scale, double v_scale,
                           hipStream_t stream) {
  const int rows = geo.num_q_heads + 2 * geo.num_kv_heads;
  const int grid = (geo.batch * geo.tokens * rows + 3) / 4;
  if (fp8) {
    prologue_kernel<true><<<grid, 256, 0, stream>>>(
        geo, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, positions,
        (const uint16_t*)wq, (const uint16_t*)wk, block_table, k_cache, v_cache,
        (uint16_t*)q_out, error_word, freqs, eps, norm_first, k_scale, v_scale);
  } else {
    prologue_kernel<false><<<grid, 256, 0, stream>>>(
        geo, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, positions,
        (const uint16_t*)wq, (const uint16_t*)wk, block_table, k_cache, v_cache,
        (uint16_t*)q_out, error_word, freqs, eps, norm_first, k_scale, v_scale);
  }
  return hipGetLastError();
}

}  // namespace lbsr
