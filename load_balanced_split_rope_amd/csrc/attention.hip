// Split attention over scheduled 64-token tiles, and the log-sum-exp merge.
//
// [A] "Why does dynamic scheduling matter in attention?" splits the KV range
// of a sequence across compute units (split-KV) in 64-token tiles; a split's
// partial result then has to be merged.  Each chunk of the schedule is one
// online-softmax pass (running max, running sum, rescaled accumulator) over
// its tiles; a sequence cut into several chunks is merged with log-sum-exp
// weights in ascending chunk order.  [A] "Two new HPC backends in the vLLM
// ecosystem": 8 query heads share each KV head, so one KV read serves the
// whole group.
//
// Mapping on CDNA4 (wave64, matrix cores):
//   * workgroup = one worker of the schedule; wave = one (KV head, block of
//     16 columns) of it at a time.
//   * S^T[64 tokens][16 cols] = K[64][128] . Q^T[128][16] with
//     v_mfma_f32_16x16x32_bf16: column j*G + h is q head h of the group for
//     new token j, so the 8 heads of the pages' model fill 8 of the 16
//     columns in a one-token step and all 16 with two new tokens per
//     sequence (multi-token decode) at no extra KV traffic; unused columns
//     are zero.  More than 16 columns (up to 64) are split into blocks of
//     16, each run by its own wave.  4 token blocks x 4 channel steps.
//   * O^T[128][16] += V^T[128][64] . P^T[64][16]: 8 channel blocks x 2 token
//     steps.  The score accumulator's lane layout is reused as the P^T operand
//     without moving data: the V page layout orders tokens to match it.
//   * every K or V fragment is one contiguous 1 KiB global read per wave
//     (16 bytes per lane), straight into the matrix-core operand registers;
//     a wave requests the next tile's K and V in one burst after P.V.
//   * FP8 E4M3 codes are widened to BF16 exactly (v_cvt_scalef32_pk_bf16_fp8
//     with scale 1); k_scale folds into the softmax scale, v_scale into the
//     output.  With FP8 scores (kQk8) the K codes feed FP8 matrix cores as
//     stored, against q's codes; q_scale then folds into the softmax scale.
//   * row max and row sum: 16 values per lane in registers, then two xor
//     shuffles across the 4 lanes that hold the same column.

#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tile_math.h"

namespace lbsr {

template <bool kFp8>
struct TileRegs {
  static constexpr int kFrags = kFp8 ? 8 : 16;  // 1 KiB fragments per K (or V) tile
  u32x4 k[kFrags];
  u32x4 v[kFrags];
};

// KV pages are read once per step: non-temporal loads stream them without
// displacing reusable lines (on MI355X these sustain ~7 TB/s against ~6.2 TB/s
// for plain loads in a pure streaming read).
template <bool kFp8>
__device__ __forceinline__ void load_frags(u32x4 (&dst)[TileRegs<kFp8>::kFrags],
                                           const u32x4* __restrict__ tile, int lane) {
#pragma unroll
  for (int f = 0; f < TileRegs<kFp8>::kFrags; ++f)
    dst[f] = __builtin_nontemporal_load(tile + f * kWave + lane);
}

// The pieces of one tile step.  Scores S^T[token][col] (lane holds tokens
// 16*tb + 4*kc + e of its column) from the K fragments and q's operand.
template <bool kFp8, bool kQk8>
__device__ __forceinline__ void tile_scores(const TileRegs<kFp8>& R, const bf16x8 (&qB)[4],
                                            const i32x8& qF, f32x4 (&S)[4]) {
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kQk8) {
      acc = mfma_fp8(k_fp8_operand(R.k[2 * tb], R.k[2 * tb + 1]), qF, acc);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 a;
        if constexpr (kFp8) {
          const u32x4 w = R.k[2 * tb + (s >> 1)];
          a = (s & 1) ? e4m3x8_to_bf16x8(w[2], w[3]) : e4m3x8_to_bf16x8(w[0], w[1]);
        } else {
          a = as_bf16x8(R.k[4 * tb + s]);
        }
        acc = mfma_bf16(a, qB[s], acc);
      }
    }
    S[tb] = acc;
  }
}

// Rows past the sequence end hold anything (even NaN): zero their V.
template <bool kFp8>
__device__ __forceinline__ void zero_v_tail(TileRegs<kFp8>& R, int rem, int kc) {
  constexpr int NF = TileRegs<kFp8>::kFrags;
  uint32_t keep[2][4];
  v_keep_masks<kFp8>(rem, kc, keep);
  if constexpr (kFp8) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) R.v[f][j] &= keep[0][j];
  } else {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) R.v[2 * db + s][j] &= keep[s][j];
  }
}

// O^T[channel][col] += V^T . P^T
template <bool kFp8>
__device__ __forceinline__ void tile_pv(const TileRegs<kFp8>& R, const bf16x8 (&pB)[2],
                                        f32x4 (&O)[8]) {
#pragma unroll
  for (int db = 0; db < 8; ++db) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 a;
      if constexpr (kFp8) {
        const u32x4 w = R.v[db];
        a = s ? e4m3x8_to_bf16x8(w[2], w[3]) : e4m3x8_to_bf16x8(w[0], w[1]);
      } else {
        a = as_bf16x8(R.v[2 * db + s]);
      }
      O[db] = mfma_bf16(a, pB[s], O[db]);
    }
  }
}

// After a tile's last P.V: request the next tile into the same registers, and
// in lockstep meet the other waves (no memory wait: the loads stay in flight).
template <bool kFp8, bool kSync>
__device__ __forceinline__ void prefetch_tile(TileRegs<kFp8>& R, const u32x4* next_k,
                                              const u32x4* next_v, int lane) {
  // keep the scheduler from hoisting the next loads above the MFMAs that
  // still read these registers (that would need a second register set)
  __builtin_amdgcn_sched_barrier(0);
  load_frags<kFp8>(R.k, next_k, lane);
  load_frags<kFp8>(R.v, next_v, lane);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kSync) {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One 64-token tile: scores, online softmax update, P.V.  `rem` = rows of the
// tile before the sequence end (1..64); the lane's column attends rows below
// rem - lag (lag = Tq - 1 - new-token index), and `tail` = Tq - 1 is the
// largest lag.  When kPrefetch, the
// next tile's K and V fragments are requested together once P.V has consumed
// this tile's registers, so they stream while the tile that follows is waited
// for and computed; with 8 waves per CU, every wave's arithmetic hides behind
// the others' loads.  (Requesting K early, right after the scores, splits each
// wave's 32 KiB request into two bursts and measured ~12% slower for BF16.)
//
// kSync: after the next tile's loads are issued, wait at a workgroup
// barrier.  The 8 waves of a workgroup (one per KV head) have the same work,
// but the CU's memory arbitration serves them unevenly: unsynchronised, the
// first wave finished at about 2/3 of the worker's time (BF16), leaving fewer
// waves -- and fewer bytes in flight -- for the rest.  In lockstep every wave
// streams until the end (split kernel 165 -> 161 us BF16, 89 -> 87 us FP8);
// a wave that waits has its next loads in flight already.  Only valid when
// every wave runs the same number of tiles (KV heads a multiple of the waves).
//
// kQk8 (FP8 cache only): the scores on FP8 matrix cores, one 16x16x128
// instruction per 16 rows, from the K codes as stored and q's codes (qF).
template <bool kFp8, bool kQk8, bool kPrefetch, bool kSync>
__device__ __forceinline__ void attend_tile(TileRegs<kFp8>& R, SoftmaxState& st,
                                            const bf16x8 (&qB)[4], const i32x8& qF, int rem,
                                            int lag, int tail, int kc, int lane,
                                            float score_scale_log2, const u32x4* next_k,
                                            const u32x4* next_v) {
  f32x4 S[4];
  tile_scores<kFp8, kQk8>(R, qB, qF, S);
  // online softmax (log2 domain); some column's last row may fall in this tile
  bf16x8 pB[2];
  softmax_tile(S, st, rem - tail < kPage, rem - lag, kc, score_scale_log2, pB);
  if (rem < kPage) zero_v_tail<kFp8>(R, rem, kc);
  tile_pv<kFp8>(R, pB, st.O);
  if constexpr (kPrefetch) prefetch_tile<kFp8, kSync>(R, next_k, next_v, lane);
}

// Two 16-column blocks of one KV head on one wave (G*Tq in 17..32): both
// read the tile's K and V registers, so a CU streams all 8 heads' tiles at
// once instead of 4 heads on two waves each.  Only one block's accumulator
// fits beside the tile in registers; the other block's O waits in the wave's
// LDS slot `o_lds` ([8][64] f32x4), its m and running sum in `other`.  The
// blocks alternate: the tile starts with the block in registers (`cur`), the
// two swap after its P.V, and the second block's accumulator stays in
// registers for the next tile.  q of both blocks is read from `q_lds`
// ([2][4][64] u32x4: block, step, lane; for FP8 scores [2][2][64], q's codes).
struct PairOther {
  float m, lsum;
};

template <bool kFp8, bool kQk8, bool kPrefetch, bool kSync>
__device__ __forceinline__ void attend_tile_pair(TileRegs<kFp8>& R, SoftmaxState& st,
                                                 PairOther& other, int& cur,
                                                 const u32x4* q_lds, f32x4* o_lds, int rem,
                                                 const int (&lag)[2], int tail, int kc, int lane,
                                                 float score_scale_log2, const u32x4* next_k,
                                                 const u32x4* next_v) {
  if (rem < kPage) zero_v_tail<kFp8>(R, rem, kc);
  const bool mask = rem - tail < kPage;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int j = half ? 1 - cur : cur;
    if (half == 1) {
      // swap the accumulators a quarter at a time: read the parked block's,
      // then park this one's at the same addresses (in order within the wave)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const f32x4 a = o_lds[(2 * qt) * kWave + lane];
        const f32x4 b = o_lds[(2 * qt + 1) * kWave + lane];
        o_lds[(2 * qt) * kWave + lane] = st.O[2 * qt];
        o_lds[(2 * qt + 1) * kWave + lane] = st.O[2 * qt + 1];
        st.O[2 * qt] = a;
        st.O[2 * qt + 1] = b;
      }
      const float m = st.m, l = st.lsum;
      st.m = other.m;
      st.lsum = other.lsum;
      other.m = m;
      other.lsum = l;
    }
    bf16x8 qB[4];
    i32x8 qF = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (kQk8) {
      const u32x4 lo = q_lds[(2 * j) * kWave + lane], hi = q_lds[(2 * j + 1) * kWave + lane];
      qF = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) qB[s] = as_bf16x8(q_lds[(4 * j + s) * kWave + lane]);
    }
    f32x4 S[4];
    tile_scores<kFp8, kQk8>(R, qB, qF, S);
    bf16x8 pB[2];
    softmax_tile(S, st, mask, rem - (j ? lag[1] : lag[0]), kc, score_scale_log2, pB);
    tile_pv<kFp8>(R, pB, st.O);
  }
  cur = 1 - cur;
  if constexpr (kPrefetch) prefetch_tile<kFp8, kSync>(R, next_k, next_v, lane);
}

// Workgroups are dispatched to the 8 XCDs round-robin (block b runs on XCD
// b % 8).  Give each XCD a contiguous run of workers instead: neighbouring
// workers' tile counts differ by at most one in a periodic pattern, and a
// contiguous run averages that pattern out, so every XCD gets the same work
// to within one tile per workgroup.
__device__ __forceinline__ int xcd_worker(int block, int num_blocks) {
  const int x = block % kXcds, j = block / kXcds;
  int start = 0;
  for (int i = 0; i < x; ++i) start += xcd_run_size(i, num_blocks);
  return start + j;
}

// The folded merge (LBSR_SCHED_FOLD_MERGE, one new token per sequence): one
// wave merges the n chunk rows of (sequence b, KV head g) -- the G heads of
// the group -- as the merge kernel does: weights 2^(lse - max) / sum per head
// over the rows, then the weighted sum of the partial rows in row order.  A
// row of the group is 32 G float4 ([16 slices of 8 channels][G heads][2
// float4]); lane l owns float4 l + 64 j, j < kNf = 32 G / 64 (one for G <= 2),
// all of head (l % 2G) / 2.  G is a power of two (the API checks), so lanes
// h, h + G, h + 2G, ... share head h and reduce with xor shuffles.  Loads are
// issued 8 lse / 16 float4 at a time, so a wave keeps them in flight.
template <int kNf>
__device__ inline void fold_merge(const Geometry& geo, const PlanPtrs& plan, int b, int g, int c0,
                                  int n, void* __restrict__ out, float* __restrict__ lse_out,
                                  int out_fp8, int lane) {
  const int G = geo.group, Hq = geo.num_q_heads;
  const size_t head0 = (size_t)g * G;
  const float* lse = plan.partial_lse + (size_t)c0 * Hq + head0;   // row r: lse[r * Hq + h]
  // 1. per head h = lane % G: max over the rows, then the sum of 2^(lse - max)
  const int h = lane % G, rsub = lane / G, rstep = kWave / G;
  float mx = -__builtin_inff();
  for (int r0 = rsub; r0 < n; r0 += 8 * rstep) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * rstep;
      x[u] = lse[(size_t)(r < n ? r : n - 1) * Hq + h];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r0 + u * rstep < n) mx = fmaxf(mx, x[u]);
  }
  for (int d = G; d < kWave; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));
  float sum = 0.f;
  for (int r0 = rsub; r0 < n; r0 += 8 * rstep) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * rstep;
      x[u] = lse[(size_t)(r < n ? r : n - 1) * Hq + h];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r0 + u * rstep < n) sum += fast_exp2(x[u] - mx);
  }
  for (int d = G; d < kWave; d <<= 1) sum += __shfl_xor(sum, d, kWave);
  if (lane < G && lse_out) lse_out[(size_t)b * Hq + head0 + lane] = (mx + __builtin_amdgcn_logf(sum)) * kLn2;

  // 2. the weighted sum over the rows, kRows rows of kNf float4 per round
  constexpr int kRows = 16 / kNf;
  const int per_row = 32 * G;                          // float4 of a group's row
  const bool fv = lane < per_row;                      // G = 1: 32 float4, lanes 32.. idle
  const int hh = (lane % (2 * G)) >> 1;                // the head of every float4 this lane owns
  const float hmx = __shfl(mx, hh, kWave);             // lane hh holds head hh's max and sum
  const float hinv = 1.0f / __shfl(sum, hh, kWave);
  const f32x4* po = (const f32x4*)plan.partial_o + ((size_t)c0 * Hq + head0) * 32 + lane;
  const size_t row_stride = (size_t)Hq * 32;           // float4 per chunk row
  f32x4 acc[kNf];
#pragma unroll
  for (int j = 0; j < kNf; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < n; r0 += kRows) {
    float lw[kRows];
    f32x4 o[kRows][kNf];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const size_t r = (size_t)(r0 + u < n ? r0 + u : n - 1);
      lw[u] = lse[r * Hq + hh];
#pragma unroll
      for (int j = 0; j < kNf; ++j) o[u][j] = fv ? po[r * row_stride + 64 * j] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      if (r0 + u < n) {
        const float w = fast_exp2(lw[u] - hmx) * hinv;
#pragma unroll
        for (int j = 0; j < kNf; ++j) acc[j] += w * o[u][j];
      }
    }
  }
  if (!fv) return;
  const size_t orow = (size_t)b * Hq + head0 + hh;
#pragma unroll
  for (int j = 0; j < kNf; ++j) {
    const int f = lane + 64 * j;
    const int d = (f / (2 * G)) * 8 + (f & 1) * 4;
    if (out_fp8) {
      *(uint32_t*)((uint8_t*)out + orow * kHeadDim + d) =
          f32x4_to_e4m3x4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
    } else {
      bf16x4 rr;
#pragma unroll
      for (int x = 0; x < 4; ++x) rr[x] = (__bf16)acc[j][x];
      *(bf16x4*)((uint16_t*)out + orow * kHeadDim + d) = rr;
    }
  }
}

// kNf for the group size G (a power of two <= 16).
__device__ inline void fold_merge_group(const Geometry& geo, const PlanPtrs& plan, int b, int g,
                                        int c0, int n, void* __restrict__ out,
                                        float* __restrict__ lse_out, int out_fp8, int lane) {
  switch (geo.group) {
    case 16: fold_merge<8>(geo, plan, b, g, c0, n, out, lse_out, out_fp8, lane); break;
    case 8: fold_merge<4>(geo, plan, b, g, c0, n, out, lse_out, out_fp8, lane); break;
    case 4: fold_merge<2>(geo, plan, b, g, c0, n, out, lse_out, out_fp8, lane); break;
    default: fold_merge<1>(geo, plan, b, g, c0, n, out, lse_out, out_fp8, lane); break;
  }
}

// A chunk's result for one lane's column (gc < G*Tq; other lanes only take
// part in the sums): the output row itself for a one-chunk sequence (BF16, or
// E4M3 codes of o / out_scale), else a partial row and its log2-sum-exp for
// the merge.
__device__ __forceinline__ void store_chunk_column(const Geometry& geo, const PlanPtrs& plan,
                                                   const f32x4 (&O)[8], float m, float lsum,
                                                   int b, int c, int g, int gc, int tok, int hl,
                                                   bool single, void* __restrict__ out,
                                                   float* __restrict__ lse_out, float out_scale,
                                                   int out_fp8, int kc) {
  const int Hq = geo.num_q_heads, G = geo.group, T = geo.tokens, GT = G * T;
  // l = 0: no row of this chunk is visible to the column (an early new
  // token whose limit lies before the chunk): an empty partial, o = 0 and
  // lse = -inf, which the merge weighs 0.  A sequence's first chunk
  // holds row 0, so a single-chunk sequence never gets here with l = 0.
  const float l = sum_xor32(sum_xor16(lsum));
  const float scale = l > 0.f ? out_scale / l : 0.f;
  const float lse2 = l > 0.f ? m + __builtin_amdgcn_logf(l) : -__builtin_inff();  // log2
  if (gc < GT) {
    const size_t orow = ((size_t)b * T + tok) * Hq + (size_t)g * G + hl;  // out / lse_out row
    if (single && out_fp8) {
      // E4M3 codes of o / out_scale (folded into scale): 4 bytes per db
      uint8_t* o = (uint8_t*)out + orow * kHeadDim + 4 * kc;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f32x4 x = O[db] * scale;
        *(uint32_t*)(o + 16 * db) = f32x4_to_e4m3x4(x[0], x[1], x[2], x[3]);
      }
      if (kc == 0 && lse_out) lse_out[orow] = lse2 * kLn2;
    } else if (single) {
      uint16_t* o = (uint16_t*)out + orow * kHeadDim + 4 * kc;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(O[db][e] * scale);
        *(bf16x4*)(o + 16 * db) = v4;
      }
      if (kc == 0 && lse_out) lse_out[orow] = lse2 * kLn2;
    } else {
      // partial row layout of (chunk c, KV group g): [16 slices of 8
      // channels][G*Tq columns][8 channels], so that any run of slices is
      // contiguous for the merge; chunk c's rows are Hq*Tq long
      const size_t HqT = (size_t)Hq * T;
      float* po = plan.partial_o + ((size_t)c * HqT + (size_t)g * GT) * kHeadDim +
                  gc * 8 + 4 * (kc & 1);
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *(f32x4*)(po + (2 * db + (kc >> 1)) * 8 * GT) = O[db] * scale;
      if (kc == 0) plan.partial_lse[(size_t)c * HqT + (size_t)g * GT + gc] = lse2;
    }
  }
}

// One worker of the schedule (this workgroup): all chunks of `worker`, every
// KV head (one wave per head, looping if Hkv > 8).
template <bool kFp8, bool kQk8, bool kSync, bool kFold>
__device__ __forceinline__ void split_worker(
    int worker, const Geometry& geo, const uint16_t* __restrict__ q_out, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const int32_t* __restrict__ block_table,
    const PlanPtrs& plan, void* __restrict__ out, float* __restrict__ lse_out,
    float score_scale_log2, float out_scale, int out_fp8, float inv_q_scale, int fold_status) {
  constexpr int kElemBytes = kFp8 ? 1 : 2;
  const int c_begin = read_invariant(plan.worker_chunk + worker);
  const int c_end = read_invariant(plan.worker_chunk + worker + 1);
  if (c_begin >= c_end) return;

  const int lane = threadIdx.x & 63;
  const int col = lane & 15;  // matrix column inside the wave's block of 16
  const int kc = lane >> 4;   // which 8-element slice of the contraction this lane feeds
  const int nwaves = blockDim.x >> 6;
  const int Hq = geo.num_q_heads, G = geo.group, T = geo.tokens;
  const int GT = G * T;              // columns of one KV head: (new token, q head) pairs
  const int ncb = (GT + 15) >> 4;    // blocks of 16 columns per KV head

  // A wave runs one (KV head, column block) at a time.  With several blocks
  // per head, the waves of one head are neighbours and read the same tiles
  // at about the same time (in lockstep), so the repeats come from L2.
  for (int vg = threadIdx.x >> 6; vg < geo.num_kv_heads * ncb; vg += nwaves) {
    const int g = vg / ncb;
    const int gc = (vg - g * ncb) * 16 + col;   // this lane's column among the head's GT
    const int tok = gc < GT ? gc / G : 0;       // its new token
    const int hl = gc - tok * G;                // and its head inside the group
    const int lag = T - 1 - tok;                // it attends rows < L - lag
    for (int c = c_begin; c < c_end; ++c) {
      const int32_t* ch = plan.chunks + 4 * (size_t)c;
      const int b = read_invariant(ch);
      const int t0 = read_invariant(ch + 1);
      const int t1 = read_invariant(ch + 2);
      // the first page's read goes out beside the sequence's length and chunk
      // count, one round trip after the chunk record
      const int32_t* bt_row = block_table + (size_t)b * geo.max_blocks;
      bool bad_page = false;
      int page = fetch_page(bt_row, t0, geo.num_pages, bad_page);
      const int L = read_invariant(plan.seq_len_eff + b);
      const int c_first = read_invariant(plan.seq_chunk + b);   // the sequence's chunks
      const int nchunks = read_invariant(plan.seq_chunk + b + 1) - c_first;
      const bool single = nchunks == 1;

      // Q^T operand: column col = q head g*G + hl of new token tok (zero past
      // the G*Tq columns in use), channels 32*s + 8*kc .. +8 for step s.
      bf16x8 qB[4];
      if (gc < GT) {
        const u32x4* qp =
            (const u32x4*)(q_out + (((size_t)b * T + tok) * Hq + (size_t)g * G + hl) * kHeadDim) +
            kc;
#pragma unroll
        for (int s = 0; s < 4; ++s) qB[s] = as_bf16x8(qp[4 * s]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) qB[s] = as_bf16x8(u32x4{0, 0, 0, 0});
      }
      SoftmaxState st;
#pragma unroll
      for (int i = 0; i < 8; ++i) st.O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      st.m = -__builtin_inff();
      st.lsum = 0.f;

      const size_t head_off = (size_t)g * geo.head_stride;
      auto tile_ptr = [&](const uint8_t* pool, int page) {
        return (const u32x4*)(pool + ((size_t)page * geo.page_stride + head_off) * kElemBytes);
      };

      TileRegs<kFp8> R;
      load_frags<kFp8>(R.k, tile_ptr(k_pool, page), lane);
      load_frags<kFp8>(R.v, tile_ptr(v_pool, page), lane);
      // q's E4M3 codes (FP8 scores), computed while the first tile streams in
      i32x8 qF = {0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (kQk8) {
        __builtin_amdgcn_sched_barrier(0);
        qF = q_fp8_operand(qB, inv_q_scale);
      }
      // all tiles but the last prefetch their successor; the last one is peeled
      // so the loop body has no conditional loads
      for (int t = t0; t < t1 - 1; ++t) {
        const int next = fetch_page(bt_row, t + 1, geo.num_pages, bad_page);
        attend_tile<kFp8, kQk8, true, kSync>(R, st, qB, qF, L - t * kPage, lag, T - 1, kc, lane,
                                             score_scale_log2, tile_ptr(k_pool, next),
                                             tile_ptr(v_pool, next));
      }
      attend_tile<kFp8, kQk8, false, false>(R, st, qB, qF, L - (t1 - 1) * kPage, lag, T - 1, kc,
                                            lane, score_scale_log2, nullptr, nullptr);
      if (bad_page && lane == 0) atomicOr(plan.error_word, (int32_t)kErrPage);
      store_chunk_column(geo, plan, st.O, st.m, st.lsum, b, c, g, gc, tok, hl, single, out,
                         lse_out, out_scale, out_fp8, kc);
      if constexpr (kFold) {
        // One new token per sequence: vg is the KV head.  A split sequence's
        // (b, g) is finished by the wave that stores its last partial: each
        // wave publishes its partial (device-scope fence), then counts it;
        // the one that brings the count to the chunk total takes the others'
        // partials (fence) and merges.  No wave waits for another.
        bool finisher = single;
        if (!single) {
          int old;
          if constexpr (kSync) {
            // Lockstep: every wave of the workgroup finishes this chunk here.
            // Each waits for its own partial stores, then one thread
            // publishes them all (one device-scope fence per chunk, not per
            // wave) and counts the chunk for the sequence.  With more KV
            // heads than waves the waves make several passes over the chunks
            // (heads p * waves + 0 .. waves - 1 in pass p); each pass has its
            // own counter, at the pass's first head: thread 0's vg.
            __shared__ int s_old;
            __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): this wave's stores done
            __syncthreads();
            if (threadIdx.x == 0) {
              __threadfence();
              int32_t* ctr = &plan.arrivals[(size_t)b * geo.num_kv_heads + vg];
              s_old = atomicAdd(ctr, 1);
              // The last arrival puts the count back to 0, so a later launch
              // over the same plan (another layer of the step) counts afresh.
              if (s_old == nchunks - 1) atomicExch(ctr, 0);
            }
            __syncthreads();
            old = s_old;
            __syncthreads();                             // s_old is rewritten next chunk
          } else {
            __threadfence();
            old = 0;
            if (lane == 0) {
              int32_t* ctr = &plan.arrivals[(size_t)b * geo.num_kv_heads + g];
              old = atomicAdd(ctr, 1);
              if (old == nchunks - 1) atomicExch(ctr, 0);   // last arrival: reset for reuse
            }
            old = __shfl(old, 0, kWave);
          }
          if (old == nchunks - 1) {
            __threadfence();
            fold_merge_group(geo, plan, b, g, c_first, nchunks, out, lse_out, out_fp8, lane);
            finisher = true;
          }
        }
        // the prologue's status of this token, folded once per sequence (decode step only)
        if (fold_status && finisher && g == 0 && lane == 0) {
          const int32_t st = plan.token_status[b];
          if (st) atomicOr(plan.error_word, st);
        }
      }
    }
  }
}

// The kernel: one workgroup per worker.  With a trace buffer it records, per
// worker, [start, end] of the 100 MHz constant clock and the hardware ids of
// the compute unit it ran on (HW_ID, XCC_ID), for load-balance analysis.
// One worker with two 16-column blocks per KV head (G*Tq in 17..32), both on
// the head's wave (attend_tile_pair): one wave per KV head, looping if
// Hkv > 8.  Each wave owns a 16 KiB slice of the dynamic LDS: q of both
// blocks (8 KiB), then the parked block's accumulator (8 KiB).
constexpr int kPairSlotU32x4 = 16 * kWave;   // u32x4 per wave

template <bool kFp8, bool kQk8, bool kSync>
__device__ __forceinline__ void split_worker_pair(
    int worker, const Geometry& geo, const uint16_t* __restrict__ q_out,
    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_table, const PlanPtrs& plan, void* __restrict__ out,
    float* __restrict__ lse_out, float score_scale_log2, float out_scale, int out_fp8,
    float inv_q_scale) {
  constexpr int kElemBytes = kFp8 ? 1 : 2;
  extern __shared__ u32x4 s_pair[];
  const int c_begin = read_invariant(plan.worker_chunk + worker);
  const int c_end = read_invariant(plan.worker_chunk + worker + 1);
  if (c_begin >= c_end) return;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int kc = lane >> 4;
  const int nwaves = blockDim.x >> 6;
  const int Hq = geo.num_q_heads, G = geo.group, T = geo.tokens;
  const int GT = G * T;
  u32x4* q_lds = s_pair + (size_t)wave * kPairSlotU32x4;
  f32x4* o_lds = (f32x4*)(q_lds + 8 * kWave);
  // this lane's column in each block: (new token, head in the group), lag
  int gc[2], tok[2], hl[2], lag[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    gc[j] = 16 * j + col;
    tok[j] = gc[j] < GT ? gc[j] / G : 0;
    hl[j] = gc[j] - tok[j] * G;
    lag[j] = T - 1 - tok[j];
  }

  for (int g = wave; g < geo.num_kv_heads; g += nwaves) {
    for (int c = c_begin; c < c_end; ++c) {
      const int32_t* ch = plan.chunks + 4 * (size_t)c;
      const int b = read_invariant(ch);
      const int t0 = read_invariant(ch + 1);
      const int t1 = read_invariant(ch + 2);
      const int32_t* bt_row = block_table + (size_t)b * geo.max_blocks;
      bool bad_page = false;
      int page = fetch_page(bt_row, t0, geo.num_pages, bad_page);
      const int L = read_invariant(plan.seq_len_eff + b);
      const int c_first = read_invariant(plan.seq_chunk + b);
      const bool single = read_invariant(plan.seq_chunk + b + 1) - c_first == 1;

      const size_t head_off = (size_t)g * geo.head_stride;
      auto tile_ptr = [&](const uint8_t* pool, int pg) {
        return (const u32x4*)(pool + ((size_t)pg * geo.page_stride + head_off) * kElemBytes);
      };
      TileRegs<kFp8> R;
      load_frags<kFp8>(R.k, tile_ptr(k_pool, page), lane);
      load_frags<kFp8>(R.v, tile_ptr(v_pool, page), lane);

      // q of both blocks (zero past the G*Tq columns) into the wave's slot,
      // as BF16 fragments or, for FP8 scores, as q's E4M3 codes
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 qB[4];
        if (gc[j] < GT) {
          const u32x4* qp = (const u32x4*)(q_out + (((size_t)b * T + tok[j]) * Hq +
                                                     (size_t)g * G + hl[j]) * kHeadDim) + kc;
#pragma unroll
          for (int s = 0; s < 4; ++s) qB[s] = as_bf16x8(qp[4 * s]);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) qB[s] = as_bf16x8(u32x4{0, 0, 0, 0});
        }
        if constexpr (kQk8) {
          const i32x8 qF = q_fp8_operand(qB, inv_q_scale);
          q_lds[(2 * j) * kWave + lane] = u32x4{(uint32_t)qF[0], (uint32_t)qF[1],
                                                (uint32_t)qF[2], (uint32_t)qF[3]};
          q_lds[(2 * j + 1) * kWave + lane] = u32x4{(uint32_t)qF[4], (uint32_t)qF[5],
                                                    (uint32_t)qF[6], (uint32_t)qF[7]};
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) q_lds[(4 * j + s) * kWave + lane] = __builtin_bit_cast(u32x4, qB[s]);
        }
      }
      // block 0 starts in registers, block 1 parked, both empty
#pragma unroll
      for (int db = 0; db < 8; ++db) o_lds[db * kWave + lane] = f32x4{0.f, 0.f, 0.f, 0.f};
      SoftmaxState st;
#pragma unroll
      for (int i = 0; i < 8; ++i) st.O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      st.m = -__builtin_inff();
      st.lsum = 0.f;
      PairOther other{-__builtin_inff(), 0.f};
      int cur = 0;

      for (int t = t0; t < t1 - 1; ++t) {
        const int next = fetch_page(bt_row, t + 1, geo.num_pages, bad_page);
        attend_tile_pair<kFp8, kQk8, true, kSync>(R, st, other, cur, q_lds, o_lds, L - t * kPage,
                                                  lag, T - 1, kc, lane, score_scale_log2,
                                                  tile_ptr(k_pool, next), tile_ptr(v_pool, next));
      }
      attend_tile_pair<kFp8, kQk8, false, false>(R, st, other, cur, q_lds, o_lds,
                                                 L - (t1 - 1) * kPage, lag, T - 1, kc, lane,
                                                 score_scale_log2, nullptr, nullptr);
      if (bad_page && lane == 0) atomicOr(plan.error_word, (int32_t)kErrPage);

      // the block in registers, then the parked one
      const int jr = cur, jp = 1 - cur;
      store_chunk_column(geo, plan, st.O, st.m, st.lsum, b, c, g, jr ? gc[1] : gc[0],
                         jr ? tok[1] : tok[0], jr ? hl[1] : hl[0], single, out, lse_out,
                         out_scale, out_fp8, kc);
#pragma unroll
      for (int db = 0; db < 8; ++db) st.O[db] = o_lds[db * kWave + lane];
      store_chunk_column(geo, plan, st.O, other.m, other.lsum, b, c, g, jp ? gc[1] : gc[0],
                         jp ? tok[1] : tok[0], jp ? hl[1] : hl[0], single, out, lse_out,
                         out_scale, out_fp8, kc);
    }
  }
}

template <bool kFp8, bool kQk8, bool kSync>
__global__ __launch_bounds__(kMaxAttnWaves * kWave) void split_attention_pair_kernel(
    Geometry geo, const uint16_t* __restrict__ q_out, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const int32_t* __restrict__ block_table, PlanPtrs plan,
    void* __restrict__ out, float* __restrict__ lse_out, float score_scale_log2,
    float out_scale, int out_fp8, float inv_q_scale, int fold_status, int64_t* __restrict__ trace) {
  (void)fold_status;
  int64_t t_start = 0;
  if (trace != nullptr && threadIdx.x == 0) t_start = (int64_t)wall_clock64();
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  split_worker_pair<kFp8, kQk8, kSync>(worker, geo, q_out, k_pool, v_pool, block_table, plan, out,
                                       lse_out, score_scale_log2, out_scale, out_fp8, inv_q_scale);
  if (trace != nullptr) {
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t* tr = trace + 4 * (size_t)worker;
      tr[0] = t_start;
      tr[1] = (int64_t)wall_clock64();
      tr[2] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_REG_HW_ID
      tr[3] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
    }
  }
}

template <bool kFp8, bool kQk8, bool kSync, bool kFold>
__global__ __launch_bounds__(kMaxAttnWaves * kWave) void split_attention_kernel(
    Geometry geo, const uint16_t* __restrict__ q_out, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const int32_t* __restrict__ block_table, PlanPtrs plan,
    void* __restrict__ out, float* __restrict__ lse_out, float score_scale_log2,
    float out_scale, int out_fp8, float inv_q_scale, int fold_status, int64_t* __restrict__ trace) {
  int64_t t_start = 0;
  if (trace != nullptr && threadIdx.x == 0) t_start = (int64_t)wall_clock64();
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  split_worker<kFp8, kQk8, kSync, kFold>(worker, geo, q_out, k_pool, v_pool, block_table, plan, out,
                                  lse_out, score_scale_log2, out_scale, out_fp8, inv_q_scale,
                                  fold_status);
  if (trace != nullptr) {
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t* tr = trace + 4 * (size_t)worker;
      tr[0] = t_start;
      tr[1] = (int64_t)wall_clock64();
      tr[2] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_REG_HW_ID
      tr[3] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
    }
  }
}

// Merge of the chunks of every sequence that has more than one.
//
// A sequence's n chunk rows (the G heads of KV group g in partial_o[c], laid
// out as 16 slices of 8 channels x G heads, plus their log2-sum-exp) are read
// in parallel: workgroup (s, g, b) owns slice run s of sequence b -- 16/S of
// the 16 slices, one contiguous 128G*4/S-byte piece of every row -- where S
// grows with n up to the grid's slice count, and rows beyond one round are
// read in further rounds.  A piece is 32G/S float4 (at most 128); a lane holds
// kP = 1 or 2 of them, so one wave instruction covers 64 kP/(32G/S) rows, and
// each lane keeps kMergeUnroll rows in flight.  The first round of row
// reads is issued before the lse are staged in LDS and turned into weights
// 2^(lse - max) / sum per head, so the two overlap.  Per-(wave, row-lane)
// sums are added in a fixed order: deterministic.
#ifndef LBSR_MERGE_WAVES
#define LBSR_MERGE_WAVES 4
#endif
#ifndef LBSR_MERGE_UNROLL
#define LBSR_MERGE_UNROLL 8
#endif
#ifndef LBSR_MERGE_LSE_UNROLL
#define LBSR_MERGE_LSE_UNROLL 8
#endif
#ifndef LBSR_MERGE_MIN_SLICES
#define LBSR_MERGE_MIN_SLICES 4
#endif
#ifndef LBSR_MERGE_MAX_SLICES
#define LBSR_MERGE_MAX_SLICES 4
#endif
constexpr int kMergeWaves = LBSR_MERGE_WAVES;
constexpr int kMergeUnroll = LBSR_MERGE_UNROLL;
constexpr int kMergeLseUnroll = LBSR_MERGE_LSE_UNROLL;

// The grid has slices x Hkv x batch workgroups (1024 for 32 sequences of 8 KV
// heads), most of them short-lived; 4 of them per CU (<= 128 VGPRs per wave)
// keep the whole grid resident at once, which measured faster than deeper
// per-thread unrolling at lower occupancy.
template <int kP>
__global__ __launch_bounds__(kMergeWaves * kWave, 4) void merge_kernel(Geometry geo, PlanPtrs plan,
                                                                    void* __restrict__ out,
                                                                    float* __restrict__ lse_out,
                                                                    int min_slices, int out_fp8,
                                                                    int fold_token_status) {
  constexpr int kThreads = kMergeWaves * kWave;
  const int slice = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int T = geo.tokens, G0 = geo.group;
  if (fold_token_status && slice == 0 && g == 0 && (int)threadIdx.x < T) {
    const int32_t st = plan.token_status[(size_t)b * T + threadIdx.x];
    if (st) atomicOr(plan.error_word, st);
  }
  const int c0 = plan.seq_chunk[b], c1 = plan.seq_chunk[b + 1];
  const int count = c1 - c0;
  if (count <= 1) return;  // written directly by the split kernel
  // A chunk row holds, per KV group, G = G0 * Tq columns (new token j, head
  // h of the group at column j*G0 + h); partial rows are Hq = Hq0 * Tq long.
  const int Hq = geo.num_q_heads * T, G = G0 * T;
  // out / lse_out row of column v of this group
  auto out_row = [&](int v) {
    const int j = v / G0;
    return ((size_t)b * T + j) * geo.num_q_heads + (size_t)g * G0 + (v - j * G0);
  };
  // Slices for this sequence: the fewest (from min_slices) whose rows all fit
  // in one round of reads, at most gridDim.x; surplus workgroups leave.
  int nslices = min_slices;
  while (nslices < (int)gridDim.x &&
         count > kMergeWaves * (kWave / (G * 32 / nslices / kP)) * kMergeUnroll)
    nslices *= 2;
  if (slice >= nslices) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const size_t head0 = (size_t)g * G;
  extern __shared__ float s_w[];                           // [count][G]: lse, then weights
  __shared__ f32x4 s_acc[kP][kThreads];                    // kP partial sums per lane

  // Loads below are unconditional (indices clamped into range, results of the
  // clamped ones discarded) so that a thread's loads issue back to back.
  // A lane holds kP float4 of a row's piece: e and e + per_lane.
  const int per_row = G * 32 / nslices;   // float4 of one row's piece (<= 64 kP)
  const int per_lane = per_row / kP;
  const int rows_per_inst = kWave / per_lane;
  const int r_sub_raw = lane / per_lane;
  const bool active = r_sub_raw < rows_per_inst;
  const int r_sub = active ? r_sub_raw : 0;
  const int e = active ? lane - r_sub_raw * per_lane : 0;   // float4 inside the piece
  // a row is [16 slices of 8 channels][G columns][2 float4]; float4 f of the
  // row (f = slice * per_row + e) holds column (f % 2G) / 2
  int hh[kP];
#pragma unroll
  for (int p = 0; p < kP; ++p) hh[p] = ((slice * per_row + e + p * per_lane) % (2 * G)) >> 1;
  const f32x4* po = (const f32x4*)plan.partial_o + head0 * 32 + slice * per_row + e;
  const int rows_per_round = kMergeWaves * rows_per_inst * kMergeUnroll;
  auto row_of = [&](int base, int u) { return base + (u * kMergeWaves + wave) * rows_per_inst + r_sub; };
  f32x4 o[kMergeUnroll][kP];
  auto load_round = [&](int base) {
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int i = min(row_of(base, u), count - 1);
#pragma unroll
      for (int p = 0; p < kP; ++p)
        o[u][p] = po[(size_t)(c0 + i) * Hq * 32 + p * per_lane];   // row c0 + i of this piece
    }
  };

  // 1. lse of every row, kMergeLseUnroll loads per thread per pass, with the first round of
  //    row reads issued right behind them.  idx = i*G + h: i by a float divide,
  //    exact since idx < 2^14 and the quotient is at least 0.5/G from an integer.
  const int nval = count * G;
  const float inv_g = 1.0f / (float)G;
  for (int base = 0; base < nval; base += kMergeLseUnroll * kThreads) {
    float v[kMergeLseUnroll];
#pragma unroll
    for (int u = 0; u < kMergeLseUnroll; ++u) {
      const int idx = min(base + tid + u * kThreads, nval - 1);
      const int i = (int)(((float)idx + 0.5f) * inv_g);
      v[u] = plan.partial_lse[(size_t)(c0 + i) * Hq + head0 + (idx - i * G)];
    }
    if (base == 0) load_round(0);
#pragma unroll
    for (int u = 0; u < kMergeLseUnroll; ++u) {
      const int idx = base + tid + u * kThreads;
      if (idx < nval) s_w[idx] = v[u];
    }
  }
  __syncthreads();
  // 2. 16 lanes per head: max and sum over the rows, then the weights in place
  for (int h2 = tid >> 4; h2 < G; h2 += kThreads / 16) {
    const int sub = tid & 15;
    float mx = -__builtin_inff();
    for (int i = sub; i < count; i += 16) mx = fmaxf(mx, s_w[i * G + h2]);
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));
    float sum = 0.f;
    for (int i = sub; i < count; i += 16) sum += fast_exp2(s_w[i * G + h2] - mx);
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, kWave);
    const float inv = 1.0f / sum;
    for (int i = sub; i < count; i += 16) s_w[i * G + h2] = fast_exp2(s_w[i * G + h2] - mx) * inv;
    if (sub == 0 && slice == 0 && lse_out)
      lse_out[out_row(h2)] = (mx + __builtin_amdgcn_logf(sum)) * kLn2;
  }
  __syncthreads();

  // 3. weighted sum of this channel slice over the rows
  f32x4 acc[kP];
#pragma unroll
  for (int p = 0; p < kP; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < count; base += rows_per_round) {
    if (base > 0) load_round(base);
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int i = row_of(base, u);
#pragma unroll
      for (int p = 0; p < kP; ++p) {
        const float wgt = (active && i < count) ? s_w[min(i, count - 1) * G + hh[p]] : 0.f;
        acc[p] += wgt * o[u][p];
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kP; ++p) s_acc[p][tid] = acc[p];
  __syncthreads();
  for (int t = tid; t < per_row; t += kThreads) {
    const int p = kP == 1 ? 0 : t / per_lane, t2 = t - p * per_lane;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < kMergeWaves; ++w)
      for (int r = 0; r < rows_per_inst; ++r) sum += s_acc[p][w * kWave + r * per_lane + t2];
    // float4 f = slice * per_row + t of the row: 8-channel slice f / 2G,
    // column (f % 2G) / 2, channels 4 * (f % 2) ..
    const int f = slice * per_row + t;
    const int bs = f / (2 * G);
    const int h3 = (f % (2 * G)) >> 1;
    const int d = bs * 8 + (f & 1) * 4;
    if (out_fp8) {
      *(uint32_t*)((uint8_t*)out + out_row(h3) * kHeadDim + d) =
          f32x4_to_e4m3x4(sum[0], sum[1], sum[2], sum[3]);
    } else {
      bf16x4 rr;
#pragma unroll
      for (int x = 0; x < 4; ++x) rr[x] = (__bf16)sum[x];
      *(bf16x4*)((uint16_t*)out + out_row(h3) * kHeadDim + d) = rr;
    }
  }
}

hipError_t launch_split_attention(const Geometry& geo, bool fp8, bool out_fp8, bool qk_fp8,
                                  bool fold, bool fold_status, int num_workers, const void* q_out,
                                  const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const PlanPtrs& plan, void* out, float* lse_out,
                                  float score_scale_log2, float out_scale, float inv_q_scale,
                                  int64_t* trace, hipStream_t stream) {
  // one wave per (KV head, 16-column block), at most 8; with two blocks per
  // head (and no folded merge, which takes one new token), one wave per head
  // runs both
  const int ncb = (geo.group * geo.tokens + 15) / 16;
  const bool pair = ncb == 2 && !fold;
  const int virt = geo.num_kv_heads * (pair ? 1 : ncb);
  const int waves = virt < kMaxAttnWaves ? virt : kMaxAttnWaves;
  // lockstep only when every wave gets the same number of them
  const bool sync = virt % waves == 0;
  const size_t lds = pair ? (size_t)waves * kPairSlotU32x4 * sizeof(u32x4) : 0;
  auto launch = [&](auto kernel) {
    kernel<<<num_workers, waves * kWave, lds, stream>>>(
        geo, (const uint16_t*)q_out, (const uint8_t*)k_cache, (const uint8_t*)v_cache,
        block_table, plan, out, lse_out, score_scale_log2, out_scale, out_fp8 ? 1 : 0,
        inv_q_scale, fold_status ? 1 : 0, trace);
  };
  auto pick = [&](auto fold_c) {
    constexpr bool F = decltype(fold_c)::value;
    if (fp8 && qk_fp8) {
      if (sync) launch(split_attention_kernel<true, true, true, F>);
      else launch(split_attention_kernel<true, true, false, F>);
    } else if (fp8) {
      if (sync) launch(split_attention_kernel<true, false, true, F>);
      else launch(split_attention_kernel<true, false, false, F>);
    } else {
      if (sync) launch(split_attention_kernel<false, false, true, F>);
      else launch(split_attention_kernel<false, false, false, F>);
    }
  };
  if (pair) {
    if (fp8 && qk_fp8) {
      if (sync) launch(split_attention_pair_kernel<true, true, true>);
      else launch(split_attention_pair_kernel<true, true, false>);
    } else if (fp8) {
      if (sync) launch(split_attention_pair_kernel<true, false, true>);
      else launch(split_attention_pair_kernel<true, false, false>);
    } else {
      if (sync) launch(split_attention_pair_kernel<false, false, true>);
      else launch(split_attention_pair_kernel<false, false, false>);
    }
  } else if (fold) {
    pick(std::true_type{});
  } else {
    pick(std::false_type{});
  }
  return hipGetLastError();
}

hipError_t launch_combine(const Geometry& geo, const PlanPtrs& plan, void* out, float* lse_out,
                          int max_chunks_per_seq, bool out_fp8, bool fold_token_status,
                          hipStream_t stream) {
  // S slices: a power of two dividing 32 with 32G/S <= 64 float4 per row
  // slice, G = group * Tq columns per (chunk, KV group), at most 64.  Where
  // that takes 16 or more slices (G > 16), a lane holds two float4 of a piece
  // at half the slices: the 4-token mix's merge went from 4096 workgroups
  // (27 us) to 2048 (19.4 us).  At 16 columns the halving (2048 -> 1024
  // workgroups) measured 1 us slower: the longest sequence's rows then fall
  // to half as many workgroups.
  const int cols = geo.group * geo.tokens;
  int slices = LBSR_MERGE_MIN_SLICES;
  while (slices < 32 && 32 * cols / slices > kWave) slices *= 2;
  const bool two = slices >= 16;
  if (two) slices /= 2;
  const int max_slices = slices > LBSR_MERGE_MAX_SLICES ? slices : LBSR_MERGE_MAX_SLICES;
  dim3 grid(max_slices, geo.num_kv_heads, geo.batch);
  const size_t lds = (size_t)max_chunks_per_seq * cols * sizeof(float);
  auto kernel = two ? merge_kernel<2> : merge_kernel<1>;
  kernel<<<grid, kMergeWaves * kWave, lds, stream>>>(geo, plan, out, lse_out, slices,
                                                     out_fp8 ? 1 : 0, fold_token_status ? 1 : 0);
  return hipGetLastError();
}

}  // namespace lbsr
