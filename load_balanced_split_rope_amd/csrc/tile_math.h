// Matrix-core and softmax pieces shared by the attention kernels (decode
// split attention and prefill), gfx950 / wave64.
//
// A K tile is the A operand of S^T[64 tokens][16 cols] = K . Q^T on
// v_mfma_f32_16x16x32_bf16 and a V tile the A operand of O^T += V^T . P^T;
// lane l = 16*kc + col holds, for token block tb, the scores of tokens
// 16*tb + 4*kc + (0..3) of column col.  The tile layout that makes every
// fragment one contiguous 1 KiB is described with the cache layout in
// include/lbsr.h.
#pragma once

#include "common.h"

namespace lbsr {

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// S^T[16 rows][16 cols] += A . B over 128 channels of E4M3 codes (gfx950
// v_mfma_f32_16x16x128_f8f6f4, no block scales).  A lane l holds 32 codes of
// row l % 16, B lane l 32 codes of column l % 16; byte j of lane group l / 16
// pairs with byte j of the same group of the other operand, so any channel
// order works if both operands use it.  Accumulator layout as mfma_bf16.
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The K operand of 16-row block tb for mfma_fp8: the tile's two FP8
// fragments 2tb and 2tb+1 (channels 32s + 8kc + j at byte 8s + j).
__device__ __forceinline__ i32x8 k_fp8_operand(u32x4 lo, u32x4 hi) {
  return i32x8{(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
               (int32_t)hi[0], (int32_t)hi[1], (int32_t)hi[2], (int32_t)hi[3]};
}

// The Q operand for mfma_fp8 from the BF16 fragments qB[s] (channels
// 32s + 8kc + j): E4M3 codes of q * inv_q_scale, rounded to fp32, then to the
// nearest code (ties to even), saturating at +-448; byte 8s + j, matching K.
__device__ __forceinline__ i32x8 q_fp8_operand(const bf16x8 (&qB)[4], float inv_q_scale) {
  i32x8 r;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)qB[s][j] * inv_q_scale;
    r[2 * s] = (int32_t)f32x4_to_e4m3x4(x[0], x[1], x[2], x[3]);
    r[2 * s + 1] = (int32_t)f32x4_to_e4m3x4(x[4], x[5], x[6], x[7]);
  }
  return r;
}

// 8 E4M3 codes (two dwords) -> 8 BF16 values, exactly.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Page id of tile t, validated without branching: a bad id reads page 0 and
// sets `bad` (reported once per chunk).
__device__ __forceinline__ int fetch_page(const int32_t* __restrict__ row, int t, int64_t num_pages,
                                          bool& bad) {
  const int p = wave_uniform(row[t]);
  const bool ok = p >= 0 && p < num_pages;
  bad |= !ok;
  return ok ? p : 0;
}

// Pairwise max / sum with lane l ^ 16 and lane l ^ 32 (VALU lane swaps, no LDS).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online-softmax state of one (chunk, KV head) pass.
struct SoftmaxState {
  f32x4 O[8];   // O^T: lane holds channels 16*db + 4*kc + e of column col
  float m;      // running max (log2 domain), uniform over the 4 lanes of a column
  float lsum;   // this lane's share of the running sum
};

// Online-softmax update with one tile's scores S (the lane's 16 scores of its
// column, see above), in the log2 domain: x = fl(c*s), p = 2^(x - m).  The
// scaled score is materialised once and used for both the max and the
// exponent, so the row that sets the max gets p = 1 exactly (a one-row
// softmax returns V bit for bit).  Rows >= lim are masked when `mask`.
// Returns P^T as the two BF16 operands of the P.V step (elements e < 4 from
// token block 2s, e >= 4 from 2s + 1).
//
// Deferred rescaling: the running max m is raised (and O and the sum
// rescaled) only when some column of the wave would otherwise see
// p > 2^8 -- so on most tiles the 32 multiplies per lane of the O rescale
// are skipped, while p stays within BF16's range and fp32 sums stay far from
// overflow.  The result is the same online softmax with a different (but
// consistent) reference max.  A column with no unmasked row yet keeps
// m = -inf; 0 then serves as the exponent base, so p and alpha are 0.
__device__ __forceinline__ void softmax_tile(const f32x4 (&S)[4], SoftmaxState& st, bool mask,
                                             int lim, int kc, float c, bf16x8 (&pB)[2]) {
  float x[16];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * tb + e] = S[tb][e] * c;
  if (mask) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (16 * tb + 4 * kc + e >= lim) x[4 * tb + e] = -__builtin_inff();
  }
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
  mx = max_xor32(max_xor16(mx));
  if (__any(mx > st.m + 8.f)) {                          // wave-uniform
    const float m_new = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - (m_new == -__builtin_inff() ? 0.f : m_new));
    st.lsum *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.O[i] *= alpha;
    st.m = m_new;
  }
  const float base = st.m == -__builtin_inff() ? 0.f : st.m;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[i] = fast_exp2(x[i] - base);
    psum += x[i];
  }
  st.lsum += psum;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) pB[s][e] = (__bf16)x[8 * s + e];
}

// Byte masks that zero the V rows at or past `rem` (rows past a sequence's
// end may hold anything, NaN included, and 0 * NaN would poison P.V).
// BF16: fragment 2*db + s, dword j holds tokens 16*(2s + j/2) + 4*kc + 2*(j%2)
// + (0, 1): keep[s][j].  FP8: dword j holds tokens 16*j + 4*kc + (0..3), one
// per byte: keep[0][j].
template <bool kFp8>
__device__ __forceinline__ void v_keep_masks(int rem, int kc, uint32_t (&keep)[2][4]) {
  if constexpr (kFp8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t mk = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * j + 4 * kc + i < rem) mk |= 0xFFu << (8 * i);
      keep[0][j] = mk;
      keep[1][j] = mk;
    }
  } else {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t0k = 16 * (2 * s + (j >> 1)) + 4 * kc + 2 * (j & 1);
        keep[s][j] = (t0k < rem ? 0xFFFFu : 0u) | (t0k + 1 < rem ? 0xFFFF0000u : 0u);
      }
  }
}

}  // namespace lbsr
