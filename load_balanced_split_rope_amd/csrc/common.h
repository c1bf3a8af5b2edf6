// Shared definitions for the lbsr HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbsr {

constexpr int kHeadDim = 128;
constexpr int kPage = 64;          // tokens per page = tokens per scheduled tile
constexpr int kTileElems = kHeadDim * kPage;
constexpr int kWave = 64;
constexpr int kMaxGroup = 16;      // q heads per KV head that one matrix-core column block holds
constexpr int kMaxColumns = 64;    // (new token, q head) pairs per KV head: 4 column blocks
constexpr int kMaxTokensPerSeq = 1 << 18;  // new tokens per sequence (prefill)

// Prefill workgroups: 8 waves, each with kPrefillBlocks blocks of 16 (token,
// head) columns (kPrefillBlocksQk8 with FP8 scores, whose operands leave room
// for a third); every K/V fragment a wave reads from LDS feeds all its blocks.
#ifndef LBSR_PREFILL_WAVES
#define LBSR_PREFILL_WAVES 8
#endif
constexpr int kPrefillWaves = LBSR_PREFILL_WAVES;
#ifndef LBSR_PREFILL_BLOCKS
#define LBSR_PREFILL_BLOCKS 2
#endif
constexpr int kPrefillBlocks = LBSR_PREFILL_BLOCKS;
constexpr int kPrefillBlocksQk8 = 3;
// (token, head) columns per workgroup; the narrower width bounds the work list
constexpr int kPrefillColumns = kPrefillWaves * 16 * kPrefillBlocks;
__host__ __device__ constexpr int prefill_columns(bool qk8) {
  return kPrefillWaves * 16 * (qk8 ? kPrefillBlocksQk8 : kPrefillBlocks);
}
static_assert(kPrefillBlocksQk8 >= kPrefillBlocks, "work lists are sized for the narrower width");
constexpr int kPrefillBuckets = 4096;  // tile-count buckets of the ragged prefill's work list
constexpr int kPrefillListOffset = 256;  // work list after a 256-byte header in its workspace
constexpr int kMergeLdsBytes = 65536;  // the merge stages chunks x columns weights in LDS
constexpr int kMaxBatch = 16384;   // the plan keeps per-sequence prefix sums in LDS
constexpr int kPlanThreads = 1024;
constexpr int kMaxAttnWaves = 8;   // waves (KV heads in flight) per attention workgroup

constexpr int kXcds = 8;           // an MI355X has 8 XCDs; workgroup i is dispatched to XCD i % 8
constexpr int kMaxXcdWeight = 65536;

enum : int32_t { kErrSeqLen = 1, kErrPage = 2, kErrPosition = 4, kErrQueryStart = 8 };

// Number of the P attention workgroups that land on XCD x (those i < P with
// i % 8 == x).  Workers are handed out so that XCD x runs a contiguous range
// of this many workers, XCD 0's first.
__host__ __device__ inline int xcd_run_size(int x, int num_workers) {
  return (num_workers - x + kXcds - 1) / kXcds;
}

// RoPE frequencies theta^(-2i/128), i < 64, computed once on the host (they
// depend only on theta) and passed by value; lane i of a prologue wave reads
// omega[i].
struct RopeFreqs {
  double omega[kHeadDim / 2];
};

// The schedule's parameters, passed by value.
struct SchedParams {
  int32_t min_len;       // shorter lengths are clamped up and flagged (a sequence holds its new tokens)
  int32_t dynamic;       // 1: length-proportional, 0: static split
  int32_t num_workers;   // P (dynamic)
  int32_t splits;        // S (static)
  int32_t weighted;      // dynamic: 1 if xcd_weight is used
  int32_t xcd_weight[kXcds];
  int32_t fold_groups;   // KV heads when the merge is folded into the split launch
                         // (the plan clears batch x fold_groups arrival counters), else 0
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Device pointers of the plan arrays inside a workspace.
struct PlanPtrs {
  int32_t* error_word;
  int32_t* cu_tiles;      // [B+1]
  int32_t* worker_chunk;  // [W+1]
  int32_t* chunks;        // [C_max][4] = seq, first tile, end tile, worker
  int32_t* seq_chunk;     // [B+1]
  int32_t* seq_len_eff;   // [B]
  int32_t* token_status;  // [B] the fused prologue's per-token error bits
  float* partial_o;       // [C_max][Hq][128]
  float* partial_lse;     // [C_max][Hq], log2 domain
  int32_t* arrivals;      // [B][Hkv] chunks done, for the folded merge
};

// Geometry every kernel needs, passed by value.
struct Geometry {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;          // Hq / Hkv
  int32_t max_blocks;     // block_table row stride
  int32_t tokens;         // new tokens per sequence (Tq); group * tokens <= kMaxGroup
  int64_t num_pages;
  int64_t page_stride;    // elements
  int64_t head_stride;    // elements
};

// ---- element offsets inside one KV tile (the library's page layout) ----
// r: token row [0,64), d: channel [0,128).  See include/lbsr.h.
__device__ __forceinline__ int k_offset_bf16(int r, int d) {
  return 512 * (4 * (r >> 4) + (d >> 5)) + 8 * (16 * ((d & 31) >> 3) + (r & 15)) + (d & 7);
}
__device__ __forceinline__ int v_offset_bf16(int r, int d) {
  const int tb = r >> 4;
  const int e = 4 * (tb & 1) + (r & 3);
  return 512 * (2 * (d >> 4) + (tb >> 1)) + 8 * (16 * ((r & 15) >> 2) + (d & 15)) + e;
}
__device__ __forceinline__ int k_offset_fp8(int r, int d) {
  const int s = d >> 5;
  return 1024 * (2 * (r >> 4) + (s >> 1)) + 16 * (16 * ((d & 31) >> 3) + (r & 15)) + 8 * (s & 1) +
         (d & 7);
}
__device__ __forceinline__ int v_offset_fp8(int r, int d) {
  const int tb = r >> 4;
  const int e = 4 * (tb & 1) + (r & 3);
  return 1024 * (d >> 4) + 16 * (16 * ((r & 15) >> 2) + (d & 15)) + 8 * (tb >> 1) + e;
}

// ---- wave64 helpers ----
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T wave_uniform(T x) {
  return __builtin_amdgcn_readfirstlane(x);
}

// A wave-uniform read of memory that no kernel writes while the reading kernel
// runs (a plan written by an earlier launch): through the constant address
// space the compiler issues it as a scalar load, counted apart from the vector
// loads, so waiting for it does not also wait for vector loads issued earlier.
template <typename T>
__device__ __forceinline__ T read_invariant(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> OCP E4M3 (E4M3FN) codes: clamp to +-448, then one round to nearest
// (ties to even).  The rounding is gfx950's packed conversion
// (v_cvt_scalef32_pk_fp8_f32, scale 1): after the clamp no value can reach its
// saturation handling, and on every fp32 value of magnitude <= 448 (both signs,
// 2^31 + 2 of them, checked exhaustively on the device) it gives the same code
// as rounding the bit pattern by hand -- 4 significant bits for normals,
// multiples of 2^-9 below 2^-6, zeros keeping their sign.  A NaN gives 0x7F
// (the clamp alone would turn it into -448).
typedef short e4m3_v2i16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e4m3_clamp(float x) { return fminf(fmaxf(x, -448.f), 448.f); }

__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
  e4m3_v2i16 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, e4m3_clamp(x), 0.f, 1.f, false);
  return __builtin_isnan(x) ? 0x7Fu : ((uint32_t)r[0] & 0xFFu);
}

// Four values -> four E4M3 codes in one little-endian word.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  e4m3_v2i16 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, e4m3_clamp(a), e4m3_clamp(b), 1.f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, e4m3_clamp(c), e4m3_clamp(d), 1.f, true);
  uint32_t w = __builtin_bit_cast(uint32_t, r);
  if (__builtin_isnan(a)) w = (w & 0xFFFFFF00u) | 0x7Fu;
  if (__builtin_isnan(b)) w = (w & 0xFFFF00FFu) | 0x7F00u;
  if (__builtin_isnan(c)) w = (w & 0xFF00FFFFu) | 0x7F0000u;
  if (__builtin_isnan(d)) w = (w & 0x00FFFFFFu) | 0x7F000000u;
  return w;
}

}  // namespace lbsr
