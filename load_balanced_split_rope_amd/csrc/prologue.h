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
// One wave per row; lane l owns the rotation pair (l, l + 64).
#pragma once

#include "common.h"

namespace lbsr {

// fp64 -> BF16 bits with a single round-to-nearest-even, from the bit pattern.
__device__ inline uint16_t f64_to_bf16_rne(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
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

__device__ inline double wave_sum_f64(double x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

// Row `row` of new token `tok` (tok = b * Tq + j for new token j of sequence
// b = seq): rows [0, Hq) are q heads, [Hq, Hq+Hkv) k heads, then v heads.
// Called by a whole wave.  A k/v row whose position or page is out of range
// skips its cache write and reports LBSR_DEV_ERR_* bits: OR-ed into
// `error_word` if given, and/or stored (0 when fine) to `token_status[tok]`
// if given -- every k/v row of a token stores the same value.
template <bool kFp8>
__device__ inline void prologue_row(
    int tok, int seq, int row, const Geometry& geo, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ positions, const uint16_t* __restrict__ wq,
    const uint16_t* __restrict__ wk, const int32_t* __restrict__ block_table,
    void* __restrict__ k_cache, void* __restrict__ v_cache, uint16_t* __restrict__ q_out,
    int32_t* __restrict__ error_word, int32_t* __restrict__ token_status, const RopeFreqs& freqs,
    double eps, int norm_first, double k_scale, double v_scale) {
#pragma clang fp contract(off)
  const int Hq = geo.num_q_heads, Hkv = geo.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int pos = positions[tok];

  const uint16_t* src;
  const uint16_t* w = nullptr;
  int kind;  // 0 = q, 1 = k, 2 = v
  int g = 0;
  if (row < Hq) {
    kind = 0;
    src = q + ((size_t)tok * Hq + row) * kHeadDim;
    w = wq;
  } else if (row < Hq + Hkv) {
    kind = 1;
    g = row - Hq;
    src = k + ((size_t)tok * Hkv + g) * kHeadDim;
    w = wk;
  } else {
    kind = 2;
    g = row - Hq - Hkv;
    src = v + ((size_t)tok * Hkv + g) * kHeadDim;
  }
  const uint16_t raw0 = src[lane], raw1 = src[lane + 64];
  double y0 = bf16_to_f64(raw0), y1 = bf16_to_f64(raw1);

  if (kind != 2) {
    const double w0 = bf16_to_f64(w[lane]), w1 = bf16_to_f64(w[lane + 64]);
    const double omega = freqs.omega[lane];
    const double a = (double)pos * omega;
    double sn, cs;
    sincos(a, &sn, &cs);
    for (int step = 0; step < 2; ++step) {
      const bool do_norm = (step == 0) == (norm_first != 0);
      if (do_norm) {
        const double ms = wave_sum_f64(y0 * y0 + y1 * y1) / (double)kHeadDim;
        const double r = sqrt(ms + eps);
        y0 = y0 / r * w0;
        y1 = y1 / r * w1;
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
    return;
  }

  // cache write of the new token's row
  int32_t flags = 0;
  int page = -1;
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
  if (flags) return;
  const int r = pos & (kPage - 1);
  const size_t base = (size_t)page * geo.page_stride + (size_t)g * geo.head_stride;
  if (!kFp8) {
    uint16_t* dst = (uint16_t*)(kind == 1 ? k_cache : v_cache) + base;
    if (kind == 1) {
      dst[k_offset_bf16(r, lane)] = f64_to_bf16_rne(y0);
      dst[k_offset_bf16(r, lane + 64)] = f64_to_bf16_rne(y1);
    } else {
      dst[v_offset_bf16(r, lane)] = raw0;  // v is BF16 already: stored as is
      dst[v_offset_bf16(r, lane + 64)] = raw1;
    }
  } else {
    uint8_t* dst = (uint8_t*)(kind == 1 ? k_cache : v_cache) + base;
    if (kind == 1) {
      dst[k_offset_fp8(r, lane)] = f64_to_e4m3_sat(y0 / k_scale);
      dst[k_offset_fp8(r, lane + 64)] = f64_to_e4m3_sat(y1 / k_scale);
    } else {
      dst[v_offset_fp8(r, lane)] = f64_to_e4m3_sat(y0 / v_scale);
      dst[v_offset_fp8(r, lane + 64)] = f64_to_e4m3_sat(y1 / v_scale);
    }
  }
}


}  // namespace lbsr
