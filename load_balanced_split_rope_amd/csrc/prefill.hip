// Prefill and chunked-prefill attention: many new tokens per sequence.
//
// [B] "Why is this good?" reports the backend on prefill and mixed batches as
// well as decode.  The step's new tokens (Tq per sequence, token j at position
// L - Tq + j, its k and v already written by the prologue) attend causally:
// token j sees rows [0, L - Tq + j].  With a prefix in the cache this is
// chunked prefill; with L = Tq it is a plain prefill.  Ragged batches give
// each sequence its own Tq through q_start (the packed rows of sequence b are
// [q_start[b], q_start[b+1])); geo.tokens is then the bound on any Tq.
//
// Mapping on CDNA4:
//   * workgroup = (sequence b, KV head g, block of 256 (token, head) columns,
//     i.e. 256/G consecutive new tokens with all G q heads of the group);
//     8 waves of two 16-column blocks each, the same matrix-core shapes as
//     the decode split kernel (S^T = K.Q^T, O^T += V^T.P^T on
//     v_mfma_f32_16x16x32_bf16); every fragment a wave reads from LDS feeds
//     both of its blocks, halving LDS traffic per flop.  With FP8 scores
//     (K as E4M3 codes, q as codes) the operands are small enough for three
//     blocks per wave: 384 columns per workgroup, a third fewer LDS and L2
//     reads per flop.
//   * the block's causal range [0, L - Tq + last token] is walked tile by
//     tile; each K/V tile is read from HBM once per workgroup, straight into
//     LDS in its fragment order (the page layout already is the operand
//     order), double-buffered: tile t+1 is requested while the waves compute
//     on tile t from LDS, and lands in the other buffer before the workgroup
//     barrier.  A BF16 tile goes there by global-to-LDS loads; an FP8 tile
//     through registers (converted to BF16 on the way for BF16 scores).
//   * one online-softmax pass per column over the whole range, so the result
//     goes straight to the output: no partials, no merge.
//   * workgroups are numbered longest-first (the blocks of the last tokens
//     see the most rows), so the dispatcher starts the long ones first.
//     Workgroups reach CUs in a fixed rotation by index, not greedily: a
//     grid that interleaves blocks of unequal length (or empty ones) leaves
//     CUs idle, each bound to the same few sequences.  A ragged batch is
//     therefore dispatched from a work list that a one-workgroup plan sorts
//     by tile count, longest first, with no empty entries (prefill_plan_kernel).

#include <type_traits>

#include "launch.h"
#include "plan.h"
#include "tile_math.h"

namespace lbsr {

// s_waitcnt operand: vmcnt(0), with expcnt and lgkmcnt left at their maxima
constexpr int kWaitVmcnt0 = 0x0F70;
// cache-policy operand of a global-to-LDS load: nt, as for the streamed tiles
constexpr int kLoadNonTemporal = 2;

// maximum with lane l ^ kXor (16 or 32), by the gfx950 lane-swap instructions
template <int kXor>
__device__ __forceinline__ float lane_maximum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = kXor == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                            : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The online softmax of one tile as softmax_tile computes it, with the score
// scale applied inside the exponent: the column max is taken over the raw
// scores and scaled once (c > 0, so fl(max s * c) = max fl(s * c): the same
// running max), and p = 2^fma(s, c, -m), one instruction per score where
// softmax_tile spends a multiply and a subtract.
//
// The running max m need not be the exact maximum: any m at or below it gives
// the same softmax (the factor 2^-m cancels between O and the sum) as long as
// no p overflows.  So once every column of the wave has a finite m, a tile
// first takes p = 2^fma(s, c, -m) against the m it has, and keeps it when no
// lane's sum of the tile's p reaches 2^16: then every p is below 2^16 (the
// tile's scores rose at most about 16 above m in the log2 domain), which
// leaves O and the sum far from fp32 overflow and keeps P's BF16 rounding
// relative, as before.  That skips the tile's max, its cross-lane reduction
// and the rescale test.  Otherwise (a score far above m, the first tile, a
// NaN or an infinity) the tile takes the full update: the max over its
// scores, and a rescale when that max is more than 8 above m.
__device__ __forceinline__ float sum16(const float (&x)[16]) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = x[2 * i] + x[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = a[2 * i] + a[2 * i + 1];
  return (a[0] + a[1]) + (a[2] + a[3]);
}

__device__ __forceinline__ void softmax_tile_fma(const f32x4 (&S)[4], SoftmaxState& st, bool mask,
                                                 int lim, int kc, float c, bf16x8 (&pB)[2]) {
  float x[16];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * tb + e] = S[tb][e];
  if (mask) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (16 * tb + 4 * kc + e >= lim) x[4 * tb + e] = -__builtin_inff();
  }
  float p[16];
  float psum = 0.f;
  bool kept = false;
  if (__all(st.m != -__builtin_inff())) {                // wave-uniform
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(__builtin_fmaf(x[i], c, -st.m));
    psum = sum16(p);
    kept = __all(psum < 65536.f);                        // false on NaN and infinity
  }
  if (!kept) {
    // IEEE maximum (NaN-propagating): a chain of v_maximum3_f32, without the
    // operand quieting that fmaxf needs; equal to fmaxf on the finite and -inf
    // scores, and a NaN score reaches the output through P either way
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, x[i]);
    mx = lane_maximum<32>(lane_maximum<16>(mx)) * c;
    if (__any(mx > st.m + 8.f)) {                        // wave-uniform
      const float m_new = fmaxf(st.m, mx);
      const float alpha = fast_exp2(st.m - (m_new == -__builtin_inff() ? 0.f : m_new));
      st.lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) st.O[i] *= alpha;
      st.m = m_new;
    }
    const float nbase = st.m == -__builtin_inff() ? 0.f : -st.m;
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(__builtin_fmaf(x[i], c, nbase));
    psum = sum16(p);
  }
  st.lsum += psum;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) pB[s][e] = (__bf16)p[8 * s + e];
}

template <bool kFp8, bool kQk8>
__global__ __launch_bounds__(kPrefillWaves * kWave) void prefill_kernel(
    Geometry geo, const uint16_t* __restrict__ q_out, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, void* __restrict__ out, float* __restrict__ lse_out,
    float score_scale_log2, float out_scale, int out_fp8, int32_t* __restrict__ error_word,
    int num_blocks_q, const int32_t* __restrict__ q_start, int total_tokens,
    const int32_t* __restrict__ work, float inv_q_scale) {
  // column blocks per wave (FP8 scores: three, whose operands fit beside them)
  constexpr int kBlocks = kQk8 ? kPrefillBlocksQk8 : kPrefillBlocks;
  constexpr int kColumns = prefill_columns(kQk8);
  constexpr int NF = kFp8 ? 8 : 16;                  // 1 KiB fragments per K (or V) tile
  constexpr int kStage = 2 * NF * kWave;             // u32x4 of one tile in HBM: K then V
  constexpr int kPerThread = kStage / (kPrefillWaves * kWave);   // 4 (BF16) or 2 (FP8)
  constexpr int kElemBytes = kFp8 ? 1 : 2;
  // FP8 cache with BF16 scores: each tile is converted to BF16 once, as it is
  // staged into LDS, instead of by each of the workgroup's waves as they read
  // it; the tile loop then runs the BF16 form.  An FP8 fragment f holds, per
  // lane, the values of BF16 fragments 2f (its low 8 bytes) and 2f + 1 (its
  // high 8 bytes), for K and for V.  With FP8 scores K stays FP8 in LDS.
  constexpr bool kCvtStage = kFp8 && !kQk8;
  constexpr bool kFp8Lds = kFp8 && !kCvtStage;       // the LDS stage holds E4M3 codes
  constexpr int NFL = kFp8Lds ? 8 : 16;              // 1 KiB fragments per K (or V) tile in LDS
  // A BF16 cache is staged by the global-to-LDS loads: each lane's 16 bytes
  // go straight to its slot (the fragment order puts lane l of a wave's 1 KiB
  // at l * 16, which is where those loads write), with no trip through
  // registers and no LDS store instructions.  The two stages are then
  // separate arrays, and the loop takes tiles in pairs so that every step
  // names its stage statically: the compiler can tell a step's LDS reads from
  // the loads filling the other stage, and waits for those only at the step's
  // end.  (With FP8 codes in LDS, for FP8 scores, the same staging measured
  // about 3% slower than staging through registers.)  Staged through
  // registers, the two stages are one array indexed by t & 1.
  constexpr bool kDma = !kFp8;
  constexpr int kStageLds = 2 * NFL * kWave;         // u32x4: 32 KiB (BF16 in LDS) / 16 KiB (FP8)

  const int G = geo.group, Hq = geo.num_q_heads;
  int qb, b, g;
  if (work) {                    // ragged batch: item blockIdx / Hkv of the sorted list
    const int item = (int)(blockIdx.x / geo.num_kv_heads);
    g = (int)(blockIdx.x % geo.num_kv_heads);
    if (item >= work[0]) return;                     // past the list: the whole workgroup leaves
    const int2 it = ((const int2*)((const char*)work + kPrefillListOffset))[item];
    b = it.x;
    qb = it.y;
  } else {
    const int per_block = geo.batch * geo.num_kv_heads;
    qb = num_blocks_q - 1 - (int)(blockIdx.x / per_block);   // last blocks first
    const int bg = (int)(blockIdx.x % per_block);
    b = bg / geo.num_kv_heads;
    g = bg - b * geo.num_kv_heads;
  }
  const int tokens_per_block = kColumns / G;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kc = lane >> 4;

  // this sequence's new tokens: T of them, at packed rows first_row + [0, T)
  int T = geo.tokens;
  size_t first_row = (size_t)b * T;
  if (q_start) {
    const int s0 = q_start[b], s1 = q_start[b + 1];
    if (s0 < 0 || s1 < s0 || s1 > total_tokens || s1 - s0 > geo.tokens) {
      if (tid == 0 && qb == 0 && g == 0 && error_word) atomicOr(error_word, (int32_t)kErrQueryStart);
      return;                                        // the whole workgroup leaves
    }
    T = s1 - s0;
    first_row = (size_t)s0;
  }
  if (qb * tokens_per_block >= T) return;            // a block past this sequence's tokens

  // length: at least the new tokens, at most the block table's reach
  const int max_len = geo.max_blocks * kPage;
  const int L_in = seq_lens[b];
  const int L = L_in < T ? T : (L_in > max_len ? max_len : L_in);
  const int tok0 = qb * tokens_per_block;
  const int tok_end = tok0 + tokens_per_block < T ? tok0 + tokens_per_block : T;
  const int limit_last = L - T + tok_end;           // rows the block's last token attends
  const int limit_first = L - T + tok0 + 1;         // and its first
  const int ntiles = (limit_last + kPage - 1) / kPage;

  // this lane's column in each of the wave's blocks: token tok0 + j, head hl
  int jt[kBlocks], hl[kBlocks], limit[kBlocks];
  bool valid[kBlocks];
  bf16x8 qB[kBlocks][4];
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb) {
    const int gc = (wave * kBlocks + cb) * 16 + col;
    const int j = gc / G;
    hl[cb] = gc - j * G;
    jt[cb] = tok0 + j;
    valid[cb] = gc < tokens_per_block * G && jt[cb] < T;
    limit[cb] = L - T + jt[cb] + 1;                 // the column attends rows < limit
    if (valid[cb]) {
      const u32x4* qp = (const u32x4*)(q_out + ((first_row + jt[cb]) * Hq + (size_t)g * G +
                                                hl[cb]) * kHeadDim) + kc;
#pragma unroll
      for (int s = 0; s < 4; ++s) qB[cb][s] = as_bf16x8(qp[4 * s]);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) qB[cb][s] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }

  const int32_t* bt_row = block_table + (size_t)b * geo.max_blocks;
  bool bad_page = false;
  auto load_tile = [&](int t, u32x4 (&dst)[kPerThread]) {
    const int p = bt_row[t];
    const bool ok = p >= 0 && p < geo.num_pages;
    bad_page |= !ok;
    const size_t base = ((size_t)(ok ? p : 0) * geo.page_stride + (size_t)g * geo.head_stride) *
                        kElemBytes;
    const u32x4* kt = (const u32x4*)(k_pool + base);
    const u32x4* vt = (const u32x4*)(v_pool + base);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int q = tid + i * kPrefillWaves * kWave;          // slot in the stage
      const u32x4* src = q < NF * kWave ? kt + q : vt + (q - NF * kWave);
      dst[i] = __builtin_nontemporal_load(src);
    }
  };
  auto store_tile = [&](u32x4* dst, const u32x4 (&src)[kPerThread]) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int q = tid + i * kPrefillWaves * kWave;          // slot in the HBM tile
      if constexpr (kCvtStage) {
        const int f = q / kWave, l = q - f * kWave;           // fragment (K, then V) and lane
        const bf16x8 lo = e4m3x8_to_bf16x8(src[i][0], src[i][1]);
        const bf16x8 hi = e4m3x8_to_bf16x8(src[i][2], src[i][3]);
        dst[(2 * f) * kWave + l] = __builtin_bit_cast(u32x4, lo);
        dst[(2 * f + 1) * kWave + l] = __builtin_bit_cast(u32x4, hi);
      } else {
        dst[q] = src[i];
      }
    }
  };
  // tile t straight into LDS: wave w's load i fills slots [i * 512 + 64 w, +64)
  auto dma_tile = [&](int t, u32x4* dst) {
    const int p = bt_row[t];
    const bool ok = p >= 0 && p < geo.num_pages;
    bad_page |= !ok;
    const size_t base = ((size_t)(ok ? p : 0) * geo.page_stride + (size_t)g * geo.head_stride) *
                        kElemBytes;
    const u32x4* kt = (const u32x4*)(k_pool + base);
    const u32x4* vt = (const u32x4*)(v_pool + base);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int q = tid + i * kPrefillWaves * kWave;
      const u32x4* src = q < NF * kWave ? kt + q : vt + (q - NF * kWave);
      __builtin_amdgcn_global_load_lds(
          (const void*)src,
          (__attribute__((address_space(3))) void*)(dst + i * kPrefillWaves * kWave + wave * kWave),
          16, 0, kLoadNonTemporal);
    }
  };

  SoftmaxState st[kBlocks];
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) st[cb].O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    st[cb].m = -__builtin_inff();
    st[cb].lsum = 0.f;
  }

  u32x4 pre[kPerThread];
  i32x8 qF[kBlocks];
  // tile 0 into stage 0; FP8 scores: q's codes for each column block,
  // computed while it streams in
  auto first_tile = [&](u32x4* dst) {
    if constexpr (kDma) dma_tile(0, dst);
    else load_tile(0, pre);
#pragma unroll
    for (int cb = 0; cb < kBlocks; ++cb) {
      qF[cb] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (kQk8) qF[cb] = q_fp8_operand(qB[cb], inv_q_scale);
    }
    if constexpr (kDma) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // this wave's loads into LDS
    else store_tile(dst, pre);
    __syncthreads();
  };
  // One tile: scores, online softmax, P.V.  Only the block's last tile can
  // reach past the sequence end, so the V-row masking is compiled into that
  // step alone (applied to every tile it costs two VALU ops per V dword).
  // cur: tile t's stage; nxt: the other, which receives tile t + 1
  auto tile_step = [&](int t, auto last_c, u32x4* cur, u32x4* nxt) {
    constexpr bool kLast = decltype(last_c)::value;
    if constexpr (!kLast) {
      if constexpr (kDma) dma_tile(t + 1, nxt);
      else load_tile(t + 1, pre);
    }
    const u32x4* kf = cur;
    const u32x4* vf = cur + NFL * kWave;

    // ---- scores: every K fragment read from LDS serves all column blocks ----
    f32x4 S[kBlocks][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int cb = 0; cb < kBlocks; ++cb) S[cb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kQk8) {
        const i32x8 a = k_fp8_operand(kf[2 * tb * kWave + lane], kf[(2 * tb + 1) * kWave + lane]);
#pragma unroll
        for (int cb = 0; cb < kBlocks; ++cb) S[cb][tb] = mfma_fp8(a, qF[cb], S[cb][tb]);
        continue;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 a;
        if constexpr (kFp8Lds) {
          const u32x4 w = kf[(2 * tb + (s >> 1)) * kWave + lane];
          a = (s & 1) ? e4m3x8_to_bf16x8(w[2], w[3]) : e4m3x8_to_bf16x8(w[0], w[1]);
        } else {
          a = as_bf16x8(kf[(4 * tb + s) * kWave + lane]);
        }
#pragma unroll
        for (int cb = 0; cb < kBlocks; ++cb) S[cb][tb] = mfma_bf16(a, qB[cb][s], S[cb][tb]);
      }
    }

    // ---- online softmax: columns' limits fall in this tile or earlier ----
    bf16x8 pB[kBlocks][2];
    const int row0 = t * kPage;
#pragma unroll
    for (int cb = 0; cb < kBlocks; ++cb)
      softmax_tile_fma(S[cb], st[cb], limit_first - row0 < kPage, limit[cb] - row0, kc,
                       score_scale_log2, pB[cb]);

    // ---- P.V; in the last tile, rows at or past the sequence end are zeroed ----
    uint32_t keep[2][4];
    if constexpr (kLast) {
      const int rem = L - row0;
      if (rem < kPage) {
        v_keep_masks<kFp8Lds>(rem, kc, keep);
      } else {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int x = 0; x < 4; ++x) keep[s][x] = ~0u;
      }
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 a;
        if constexpr (kFp8Lds) {
          u32x4 w = vf[db * kWave + lane];
          if constexpr (kLast) {
#pragma unroll
            for (int x = 0; x < 4; ++x) w[x] &= keep[0][x];
          }
          a = s ? e4m3x8_to_bf16x8(w[2], w[3]) : e4m3x8_to_bf16x8(w[0], w[1]);
        } else {
          u32x4 w = vf[(2 * db + s) * kWave + lane];
          if constexpr (kLast) {
#pragma unroll
            for (int x = 0; x < 4; ++x) w[x] &= keep[s][x];
          }
          a = as_bf16x8(w);
        }
#pragma unroll
        for (int cb = 0; cb < kBlocks; ++cb)
          st[cb].O[db] = mfma_bf16(a, pB[cb][s], st[cb].O[db]);
      }
    }
    if constexpr (!kLast) {
      if constexpr (kDma) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      else store_tile(nxt, pre);
      __syncthreads();
    }
  };
  if constexpr (kDma) {
    __shared__ u32x4 s_kv0[kStageLds];
    __shared__ u32x4 s_kv1[kStageLds];
    first_tile(s_kv0);
    // tiles in pairs (stage 0, then stage 1), the last one peeled
    int t = 0;
    for (; t + 2 < ntiles; t += 2) {
      tile_step(t, std::false_type{}, s_kv0, s_kv1);
      tile_step(t + 1, std::false_type{}, s_kv1, s_kv0);
    }
    if (t + 1 < ntiles) {
      tile_step(t, std::false_type{}, s_kv0, s_kv1);
      tile_step(t + 1, std::true_type{}, s_kv1, s_kv0);
    } else {
      tile_step(t, std::true_type{}, s_kv0, s_kv1);
    }
  } else {
    __shared__ u32x4 s_kv[2][kStageLds];
    first_tile(s_kv[0]);
    for (int t = 0; t + 1 < ntiles; ++t)
      tile_step(t, std::false_type{}, s_kv[t & 1], s_kv[(t & 1) ^ 1]);
    tile_step(ntiles - 1, std::true_type{}, s_kv[(ntiles - 1) & 1], s_kv[ntiles & 1]);
  }
  if (bad_page && error_word) atomicOr(error_word, (int32_t)kErrPage);

  // ---- output ----
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb) {
    const float l = sum_xor32(sum_xor16(st[cb].lsum));
    const float scale = l > 0.f ? out_scale / l : 0.f;
    if (!valid[cb]) continue;
    const size_t orow = (first_row + jt[cb]) * Hq + (size_t)g * G + hl[cb];
    if (out_fp8) {
      uint8_t* o = (uint8_t*)out + orow * kHeadDim + 4 * kc;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f32x4 x = st[cb].O[db] * scale;
        *(uint32_t*)(o + 16 * db) = f32x4_to_e4m3x4(x[0], x[1], x[2], x[3]);
      }
    } else {
      uint16_t* o = (uint16_t*)out + orow * kHeadDim + 4 * kc;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(st[cb].O[db][e] * scale);
        *(bf16x4*)(o + 16 * db) = v4;
      }
    }
    if (kc == 0 && lse_out)
      lse_out[orow] = (l > 0.f ? st[cb].m + __builtin_amdgcn_logf(l) : -__builtin_inff()) * kLn2;
  }
  if (tid == 0 && L != L_in && error_word && qb == 0 && g == 0)
    atomicOr(error_word, (int32_t)kErrSeqLen);
}

// The work list of a prefill (ragged, or uniform with q_start null): every
// (sequence, block of new tokens) with at least one token, grouped by
// sequence and longest first.  A sequence's key is its longest item's tile
// count (the rows its last token attends, in 64-row tiles); a counting sort
// over key buckets (tiles >> shift) orders the sequences longest first, and
// each sequence's items follow each other from its last block (the longest)
// down to its first.  The blocks of one sequence read the same prefix tiles,
// and the attention grid puts an item's KV heads on consecutive workgroups
// (head h of every item on the same XCD when Hkv = 8), so neighbouring items
// of one sequence meet in their XCD's L2.  One 1024-thread workgroup:
// per-sequence item counts, their prefix sums and each sequence's first slot
// in LDS (2 batch + 1 ints); thread t places items t, t + 1024, ... (its
// sequence by binary search over the prefix sums).  Layout of `work`: [0]
// item count, then from byte kPrefillListOffset int2 (sequence, block)
// pairs, at most max_items of them.  The order of sequences within a bucket
// is arrival order; it decides only which workgroup runs an item, not any
// result.
__device__ inline bool ragged_range(const int32_t* q_start, const int32_t* seq_lens, int b,
                                    int total_tokens, int bound, int max_len, int& T, int& L) {
  // no q_start: every sequence has `bound` new tokens (the uniform call)
  const int s0 = q_start ? q_start[b] : b * bound;
  const int s1 = q_start ? q_start[b + 1] : s0 + bound;
  if (s0 < 0 || s1 < s0 || s1 > total_tokens || s1 - s0 > bound) return false;
  T = s1 - s0;
  const int L_in = seq_lens[b];
  L = L_in < T ? T : (L_in > max_len ? max_len : L_in);
  return true;
}

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(
    Geometry geo, const int32_t* __restrict__ q_start, const int32_t* __restrict__ seq_lens,
    int total_tokens, int32_t* __restrict__ work, int max_items, int shift, int columns,
    int32_t* __restrict__ error_word) {
  extern __shared__ int s_dyn[];
  int* s_cu = s_dyn;                                // batch + 1: items before each sequence
  int* s_first = s_dyn + geo.batch + 1;             // batch: each sequence's first list slot
  __shared__ int s_bucket[kPrefillBuckets];
  __shared__ int s_wave[kPlanThreads / kWave + 1];
  const int tid = threadIdx.x, B = geo.batch;
  const int tpb = columns / geo.group;               // new tokens per block
  const int max_len = geo.max_blocks * kPage;
  // bucket of a sequence with T new tokens and L rows: its longest item's tile count
  auto bucket_of = [&](int T, int L) {
    const int tiles = (L + kPage - 1) / kPage;      // the last new token attends all L rows
    const int k = tiles >> shift;
    return kPrefillBuckets - 1 - (k < kPrefillBuckets ? k : kPrefillBuckets - 1);  // longest first
  };
  // items (blocks of new tokens) per sequence; none for a malformed range
  bool bad = false;
  for (int i = tid; i < kPrefillBuckets; i += kPlanThreads) s_bucket[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kPlanThreads) {
    int T, L;
    const bool ok = ragged_range(q_start, seq_lens, b, total_tokens, geo.tokens, max_len, T, L);
    bad |= !ok;
    const int n = ok ? (T + tpb - 1) / tpb : 0;
    s_cu[b] = n;
    if (n > 0) atomicAdd(&s_bucket[bucket_of(T, L)], n);
  }
  __syncthreads();
  int carry = 0;                                    // exclusive prefix sums, 1024 at a time
  for (int base = 0; base < B; base += kPlanThreads) {
    const int b = base + tid;
    const int n = b < B ? s_cu[b] : 0;
    int sum = 0;
    const int incl = block_inclusive_scan(n, s_wave, sum);
    if (b < B) s_cu[b] = carry + incl - n;
    carry += sum;
  }
  if (tid == 0) s_cu[B] = carry;
  // exclusive offsets over the buckets: thread t owns buckets [4t, 4t + 4)
  constexpr int kPer = kPrefillBuckets / kPlanThreads;
  int local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) local += s_bucket[kPer * tid + i];
  int total = 0;
  int off = block_inclusive_scan(local, s_wave, total) - local;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = s_bucket[kPer * tid + i];
    s_bucket[kPer * tid + i] = off;
    off += c;
  }
  __syncthreads();
  const int N = carry;
  // each sequence takes a run of slots in its bucket
  for (int b = tid; b < B; b += kPlanThreads) {
    const int n = s_cu[b + 1] - s_cu[b];
    if (n > 0) {
      int T, L;
      ragged_range(q_start, seq_lens, b, total_tokens, geo.tokens, max_len, T, L);
      s_first[b] = atomicAdd(&s_bucket[bucket_of(T, L)], n);
    }
  }
  __syncthreads();
  // item i -> (sequence, block): the last b with s_cu[b] <= i (empty sequences skipped)
  int2* list = (int2*)((char*)work + kPrefillListOffset);
  for (int i = tid; i < N; i += kPlanThreads) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_cu[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int b = lo, qb = i - s_cu[b], n = s_cu[b + 1] - s_cu[b];
    const int pos = s_first[b] + (n - 1 - qb);      // the sequence's last block first
    if (pos < max_items) list[pos] = make_int2(b, qb);
  }
  // overlapping ranges (a malformed q_start) can give more items than the list holds
  if (tid == 0) work[0] = N < max_items ? N : max_items;
  if (error_word && (bad || (tid == 0 && N > max_items)))
    atomicOr(error_word, (int32_t)kErrQueryStart);
}

// The plan's LDS at the batch limit: counts and prefix sums (batch + 1), first
// slots (batch), the buckets and the scan's per-wave sums, within gfx950's 160 KiB.
static_assert(sizeof(int) * ((2 * (size_t)kMaxBatch + 1) + kPrefillBuckets +
                             (kPlanThreads / kWave + 1)) <= 160 * 1024,
              "prefill plan LDS exceeds 160 KiB at kMaxBatch");

int prefill_blocks_q(const Geometry& geo, int columns) {
  const int per = columns / geo.group;
  return (geo.tokens + per - 1) / per;
}

int prefill_max_items(const Geometry& geo, int total_tokens, int columns) {
  const int tpb = columns / geo.group;
  return (total_tokens + tpb - 1) / tpb + geo.batch;
}

hipError_t launch_prefill(const Geometry& geo, bool fp8, bool out_fp8, const void* q_out,
                          const void* k_cache, const void* v_cache, const int32_t* block_table,
                          const int32_t* seq_lens, void* out, float* lse_out,
                          float score_scale_log2, float out_scale, int32_t* error_word,
                          const int32_t* q_start, int total_tokens, int32_t* work, bool qk_fp8,
                          float inv_q_scale, hipStream_t stream) {
  const int columns = prefill_columns(fp8 && qk_fp8);
  const int nqb = prefill_blocks_q(geo, columns);
  size_t grid = (size_t)nqb * geo.batch * geo.num_kv_heads;
  if (work) {
    // at most the entries the workspace was sized for (the narrower width)
    const int max_items = prefill_max_items(geo, total_tokens, columns);
    int shift = 0;
    while ((geo.max_blocks >> shift) >= kPrefillBuckets) ++shift;
    const size_t lds = sizeof(int) * (2 * (size_t)geo.batch + 1);
    prefill_plan_kernel<<<1, kPlanThreads, lds, stream>>>(geo, q_start, seq_lens, total_tokens,
                                                           work, max_items, shift, columns,
                                                           error_word);
    grid = (size_t)max_items * geo.num_kv_heads;
  }
  auto launch = [&](auto kernel) {
    kernel<<<(unsigned)grid, kPrefillWaves * kWave, 0, stream>>>(
        geo, (const uint16_t*)q_out, (const uint8_t*)k_cache, (const uint8_t*)v_cache,
        block_table, seq_lens, out, lse_out, score_scale_log2, out_scale, out_fp8 ? 1 : 0,
        error_word, nqb, q_start, total_tokens, work, inv_q_scale);
  };
  if (fp8 && qk_fp8) launch(prefill_kernel<true, true>);
  else if (fp8) launch(prefill_kernel<true, false>);
  else launch(prefill_kernel<false, false>);
  return hipGetLastError();
}

}  // namespace lbsr
