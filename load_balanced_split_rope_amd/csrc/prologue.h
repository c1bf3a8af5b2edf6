// Fused prologue device code: RoPE + QK-Norm on one row (one q or k head of
// one new token) or the copy/quantisation of one v row, and the cache write.
//
// [A] "Why does dynamic scheduling matter in attention?" and [B] "Code
// analysis 2" (see include/lbsr.h for the sources): the rotation, the
// normalisation and the cache write are one pass, so q/k are read once and
// written once.  Readings: rotate-half RoPE over all 128 channels with
// frequency theta^(-2i/128); RoPE before RMSNorm unless norm_first; RMSNorm
// x / sqrt(mean(x^2) + eps) * w with one weight vector for q and one for k;
// v is stored unchanged (BF16) or quantised (FP8).
//
// The work is tiny (a few MB per step) and latency bound, so it is computed
// in fp64 (full rate on CDNA4) with contraction off, and every stored value is
// rounded once from fp64: the stored bits then equal the exact result's
// rounding except within ~1e-15 relative of a rounding midpoint.  The
// frequencies come precomputed (RopeFreqs): an fp64 pow per lane was the
// largest single step of the chain.
//
// A wave runs consecutive rows of one token; lane l owns the rotation pair
// (l, l + 64).
#pragma once

#include "common.h"

namespace lbsr {

// fp64 -> BF16 bits with a single round-to-nearest-even, from the bit pattern.
__device__ inline uint16_t f64_to_bf16_rne(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  const uint32_t biased = (uint32_t)(mag >> 52);
  if (biased >= 1023 - 126 && biased <= 1023 + 127) {
    // BF16-normal range: round the magnitude's bit pattern at its 45th bit
    // (half minus one, plus the kept LSB: ties to even).  A carry moves into
    // the exponent field, and past the largest finite value gives infinity.
    const uint64_t r = mag + ((1ull << 44) - 1) + ((mag >> 45) & 1);
    return (uint16_t)((uint32_t)(u >> 48 & 0x8000) | (uint32_t)((r >> 45) - (896u << 7)));
  }
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  const int exp = (int)((u >> 52) & 0x7FF);
  const uint64_t mant = u & 0xFFFFFFFFFFFFFull;
  if (exp == 0x7FF) return (uint16_t)(mant ? 0x7FC0 : (sign | 0x7F80));
  if (exp == 0) return (uint16_t)sign;  // fp64 subnormals are below half of 2^-133
  int e = exp - 1023;
  const uint64_t sig = mant | (1ull << 52);  // value = sig * 2^(e - 52)
  if (e >= -126) {
    uint64_t q = sig >> 45;                  // 8 significant bits
    const uint64_t rem = sig & ((1ull << 45) - 1), half = 1ull << 44;
    if (rem > half || (rem == half && (q & 1))) q++;
    if (q == 256) { q = 128; e++; }
    if (e > 127) return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | (uint32_t)((e + 127) << 7) | (uint32_t)(q & 127));
  }
  // subnormal BF16: multiples of 2^-133, value / 2^-133 = sig * 2^(e + 81)
  const int s = -(e + 81);                   // > 45
  if (s >= 64) return (uint16_t)sign;
  uint64_t q = sig >> s;
  const uint64_t rem = sig & ((1ull << s) - 1), half = 1ull << (s - 1);
  if (rem > half || (rem == half && (q & 1))) q++;
  return (uint16_t)(sign | (uint32_t)q);     // q == 128 encodes the smallest normal
}

// fp64 -> OCP E4M3 (E4M3FN) code: clamp to +-448, then one RNE step.
__device__ inline uint8_t f64_to_e4m3_sat(double x) {
  if (__builtin_isnan(x)) return 0x7F;
  x = fmin(fmax(x, -448.0), 448.0);
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 63) << 7;
  const int exp = (int)((u >> 52) & 0x7FF);
  if (exp == 0) return (uint8_t)sign;
  int e = exp - 1023;
  const uint64_t sig = (u & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  if (e >= -6) {
    uint64_t q = sig >> 49;                  // 4 significant bits
    const uint64_t rem = sig & ((1ull << 49) - 1), half = 1ull << 48;
    if (rem > half || (rem == half && (q & 1))) q++;
    if (q == 16) { q = 8; e++; }             // cannot pass 448 after the clamp
    return (uint8_t)(sign | (uint32_t)((e + 7) << 3) | (uint32_t)(q & 7));
  }
  // subnormal: multiples of 2^-9, value / 2^-9 = sig * 2^(e - 43)
  const int s = 43 - e;                      // > 49
  if (s >= 64) return (uint8_t)sign;
  uint64_t q = sig >> s;
  const uint64_t rem = sig & ((1ull << s) - 1), half = 1ull << (s - 1);
  if (rem > half || (rem == half && (q & 1))) q++;
  return (uint8_t)(sign | (uint32_t)q);      // q == 8 encodes the smallest normal
}

__device__ inline double bf16_to_f64(uint16_t b) {
  return (double)__uint_as_float((uint32_t)b << 16);
}

// One fp64 value moved across lanes by a DPP pattern (both halves alike).
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, kCtrl, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), kCtrl, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the wave, every lane receiving it: the xor butterfly at distances
// 32, 16, 8, 4, 2, 1 (each lane adds its partner's value; the two partners
// add the same pair, so they stay equal).  No step goes through LDS:
// distances 32 and 16 use gfx950's permlane swaps (their two outputs are the
// lower and the upper lane's value), 8 and 4 a rotation inside the 16-lane
// row (by 8 it is the xor; by 4 it matches the xor once the values repeat
// every 8 lanes), 2 and 1 a quad permutation.
__device__ inline double wave_sum_f64(double x) {
#pragma clang fp contract(off)
  {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32),
                                                     false, false);
    x = __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]) +
        __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
  }
  {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32),
                                                     false, false);
    x = __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]) +
        __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
  }
  x = x + dpp_f64<0x128>(x);   // row_ror:8
  x = x + dpp_f64<0x124>(x);   // row_ror:4
  x = x + dpp_f64<0x4E>(x);    // quad_perm [2,3,0,1]
  x = x + dpp_f64<0xB1>(x);    // quad_perm [1,0,3,2]
  return x;
}

// Rows [row_begin, row_end) of new token `tok` (tok = b * Tq + j for new
// token j of sequence b = seq); rows [0, Hq) are q heads, [Hq, Hq+Hkv) k
// heads, then v heads.  Called by a whole wave.  The rotation angle depends
// only on the position and the channel pair, so its sine and cosine are
// computed once for the run, as are the norm weights and the cache slot.
// A k/v row whose position or page is out of range skips its cache write and
// reports LBSR_DEV_ERR_* bits: OR-ed into `error_word` if given, and/or
// stored (0 when fine) to `token_status[tok]` if given -- every run holding
// k/v rows of a token stores the same value.  kOneRow: every run is a single
// row (row_end = row_begin + 1), the decode-sized case, compiled without the
// loop.
template <bool kFp8, bool kOneRow>
__device__ inline void prologue_rows(
    int tok, int seq, int row_begin, int row_end, const Geometry& geo,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ positions,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const int32_t* __restrict__ block_table, void* __restrict__ k_cache,
    void* __restrict__ v_cache, uint16_t* __restrict__ q_out, int32_t* __restrict__ error_word,
    int32_t* __restrict__ token_status, const RopeFreqs& freqs, double eps, int norm_first,
    double k_scale, double v_scale) {
#pragma clang fp contract(off)
  const int Hq = geo.num_q_heads, Hkv = geo.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int pos = positions[tok];
  if (kOneRow) row_end = row_begin + 1;

  // the row's source: q heads, then k heads, then v heads of this token
  auto source = [&](int row) -> const uint16_t* {
    if (row < Hq) return q + ((size_t)tok * Hq + row) * kHeadDim;
    if (row < Hq + Hkv) return k + ((size_t)tok * Hkv + (row - Hq)) * kHeadDim;
    return v + ((size_t)tok * Hkv + (row - Hq - Hkv)) * kHeadDim;
  };
  const uint16_t* src = source(row_begin);
  uint16_t next0 = src[lane], next1 = src[lane + 64];

  double sn = 0.0, cs = 1.0;
  double wq0 = 0.0, wq1 = 0.0, wk0 = 0.0, wk1 = 0.0;
  if (row_begin < Hq) {
    wq0 = bf16_to_f64(wq[lane]);
    wq1 = bf16_to_f64(wq[lane + 64]);
  }
  if (row_begin < Hq + Hkv && row_end > Hq) {
    wk0 = bf16_to_f64(wk[lane]);
    wk1 = bf16_to_f64(wk[lane + 64]);
  }
  if (row_begin < Hq + Hkv) sincos((double)pos * freqs.omega[lane], &sn, &cs);

  // the cache slot of the token's k/v rows
  int32_t flags = 0;
  int page = -1;
  if (row_end > Hq) {
    if (pos < 0 || pos >= geo.max_blocks * kPage) {
      flags = kErrPosition;
    } else {
      page = block_table[(size_t)seq * geo.max_blocks + (pos >> 6)];
      if (page < 0 || page >= geo.num_pages) flags = kErrPage;
    }
    if (lane == 0) {
      if (token_status) token_status[tok] = flags;
      if (error_word && flags) atomicOr(error_word, flags);
    }
  }
  const int slot_row = pos & (kPage - 1);

  for (int row = row_begin; row < row_end; ++row) {
    const uint16_t raw0 = next0, raw1 = next1;
    if (!kOneRow && row + 1 < row_end) {     // the next row's loads, ahead of this row's math
      const uint16_t* nsrc = source(row + 1);
      next0 = nsrc[lane];
      next1 = nsrc[lane + 64];
    }
    const int kind = row < Hq ? 0 : (row < Hq + Hkv ? 1 : 2);   // q, k, v
    double y0 = bf16_to_f64(raw0), y1 = bf16_to_f64(raw1);
    if (kind != 2) {
      const double w0 = kind == 0 ? wq0 : wk0, w1 = kind == 0 ? wq1 : wk1;
      for (int step = 0; step < 2; ++step) {
        const bool do_norm = (step == 0) == (norm_first != 0);
        if (do_norm) {
          const double ms = wave_sum_f64(y0 * y0 + y1 * y1) / (double)kHeadDim;
          const double inv = 1.0 / sqrt(ms + eps);
          y0 = y0 * inv * w0;
          y1 = y1 * inv * w1;
        } else {
          const double r0 = y0 * cs - y1 * sn;
          const double r1 = y1 * cs + y0 * sn;
          y0 = r0;
          y1 = r1;
        }
      }
    }
    if (kind == 0) {
      uint16_t* dst = q_out + ((size_t)tok * Hq + row) * kHeadDim;
      dst[lane] = f64_to_bf16_rne(y0);
      dst[lane + 64] = f64_to_bf16_rne(y1);
      continue;
    }
    if (flags) continue;
    const int g = kind == 1 ? row - Hq : row - Hq - Hkv;
    const size_t base = (size_t)page * geo.page_stride + (size_t)g * geo.head_stride;
    if (!kFp8) {
      uint16_t* dst = (uint16_t*)(kind == 1 ? k_cache : v_cache) + base;
      if (kind == 1) {
        dst[k_offset_bf16(slot_row, lane)] = f64_to_bf16_rne(y0);
        dst[k_offset_bf16(slot_row, lane + 64)] = f64_to_bf16_rne(y1);
      } else {
        dst[v_offset_bf16(slot_row, lane)] = raw0;  // v is BF16 already: stored as is
        dst[v_offset_bf16(slot_row, lane + 64)] = raw1;
      }
    } else {
      uint8_t* dst = (uint8_t*)(kind == 1 ? k_cache : v_cache) + base;
      if (kind == 1) {
        dst[k_offset_fp8(slot_row, lane)] = f64_to_e4m3_sat(y0 / k_scale);
        dst[k_offset_fp8(slot_row, lane + 64)] = f64_to_e4m3_sat(y1 / k_scale);
      } else {
        dst[v_offset_fp8(slot_row, lane)] = f64_to_e4m3_sat(y0 / v_scale);
        dst[v_offset_fp8(slot_row, lane + 64)] = f64_to_e4m3_sat(y1 / v_scale);
      }
    }
  }
}

// Sequence of packed new token `tok` in a ragged batch: the last b with
// q_start[b] <= tok.  Any q_start contents give an index in [0, batch).
__device__ inline int seq_of_token(const int32_t* __restrict__ q_start, int batch, int tok) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= tok) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// How many runs each token's rows are cut into: enough waves to fill the GPU
// a few times over (one row per wave when the tokens are few, as in decode),
// a whole token per wave when they are many, as in prefill.
inline int prologue_runs_per_token(int tokens, int rows) {
  constexpr int kTargetWaves = 32768;
  const int runs = (kTargetWaves + tokens - 1) / (tokens > 0 ? tokens : 1);
  return runs < 1 ? 1 : (runs > rows ? rows : runs);
}

// Run `i` of `runs` covers rows [i * rows / runs, (i + 1) * rows / runs).
__device__ inline int prologue_run_begin(int i, int runs, int rows) { return i * rows / runs; }

}  // namespace lbsr
