// Host-side launchers of the lbsr kernels (one per kernel file).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace lbsr {

// num_tokens: batch * Tq, or the packed count of a ragged batch (q_start
// non-null: token -> sequence by binary search).
hipError_t launch_prologue(const Geometry& geo, bool fp8, const void* q, const void* k,
                           const void* v, const int32_t* positions, const void* wq,
                           const void* wk, const int32_t* block_table, void* k_cache,
                           void* v_cache, void* q_out, int32_t* error_word, const RopeFreqs& freqs,
                           double eps, int norm_first, double k_scale, double v_scale,
                           int num_tokens, const int32_t* q_start, hipStream_t stream);

hipError_t launch_plan(const int32_t* seq_lens, int batch, int max_blocks, const SchedParams& sp,
                       const PlanPtrs& plan, hipStream_t stream);

// qk_fp8 (with an FP8 cache): q quantised with inv_q_scale, scores on FP8
// matrix cores; score_scale_log2 then includes q_scale.
// fold: merge split sequences inside this launch (one new token per
// sequence); fold_status: also fold the prologue's per-token status words
// into the error word (decode step).
hipError_t launch_split_attention(const Geometry& geo, bool fp8, bool out_fp8, bool qk_fp8,
                                  bool fold, bool fold_status, int num_workers, const void* q_out,
                                  const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const PlanPtrs& plan, void* out, float* lse_out,
                                  float score_scale_log2, float out_scale, float inv_q_scale,
                                  int64_t* trace, hipStream_t stream);

// out_fp8: `out` holds E4M3 codes of the merged values (which the split
// kernel already divided by the output scale).
// fold_token_status: also OR plan.token_status (written by the fused
// plan + prologue launch of the same step) into the error word.
hipError_t launch_combine(const Geometry& geo, const PlanPtrs& plan, void* out, float* lse_out,
                          int max_chunks_per_seq, bool out_fp8, bool fold_token_status,
                          hipStream_t stream);

// q_start non-null: ragged batch, sequence b's new tokens at packed rows
// [q_start[b], q_start[b+1]) of total_tokens; geo.tokens bounds every count.
// A plan launch first writes the longest-first work list into `work`
// (kPrefillListOffset + 8 * prefill_max_items bytes).
hipError_t launch_prefill(const Geometry& geo, bool fp8, bool out_fp8, const void* q_out,
                          const void* k_cache, const void* v_cache, const int32_t* block_table,
                          const int32_t* seq_lens, void* out, float* lse_out,
                          float score_scale_log2, float out_scale, int32_t* error_word,
                          const int32_t* q_start, int total_tokens, int32_t* work, bool qk_fp8,
                          float inv_q_scale, hipStream_t stream);

// Work-list entries a ragged prefill may need: one per block of new tokens,
// blocks of `columns` (token, head) columns (kPrefillColumns bounds them all).
int prefill_max_items(const Geometry& geo, int total_tokens, int columns = kPrefillColumns);

hipError_t launch_plan_prologue(const int32_t* seq_lens, const SchedParams& sp,
                                const PlanPtrs& plan, const Geometry& geo,
                                bool fp8, const void* q, const void* k, const void* v,
                                const int32_t* positions, const void* wq, const void* wk,
                                const int32_t* block_table, void* k_cache, void* v_cache,
                                void* q_out, const RopeFreqs& freqs, double eps, int norm_first,
                                double k_scale, double v_scale, hipStream_t stream);

// Streaming-read probe (measurement only): `bytes` must be a multiple of
// stream_read_block_bytes(); sink holds one word per workgroup.  mode 0: the
// split kernel's load pattern; 1: a plain grid-wide sweep.
int64_t stream_read_block_bytes();
hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, int mode,
                              uint32_t* sink, hipStream_t stream);

// Cache layout conversion: pack (rows -> tiles) or unpack (tiles -> rows) of
// every (page, KV head) tile; strides in elements, checked on the host.
hipError_t launch_pack(bool fp8, bool v, bool pack, const void* src, void* dst, int64_t num_pages,
                       int num_kv_heads, int64_t tile_page_stride, int64_t tile_head_stride,
                       int64_t row_page_stride, int64_t row_token_stride, int64_t row_head_stride,
                       hipStream_t stream);

}  // namespace lbsr
