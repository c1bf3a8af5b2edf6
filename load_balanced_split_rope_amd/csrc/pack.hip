// Conversion between a row-major paged cache and the library's tile layout.
//
// [A] "Why does dynamic scheduling matter in attention?" fixes the 64-token
// tile as the unit in which the cache is read; the order of the elements
// inside a tile is this library's own (include/lbsr.h), chosen so that every
// K or V fragment is one contiguous 1 KiB read in matrix-core operand order.
// A caller whose cache is a plain row-major paged array -- per page, 64 token
// rows of 128 channels for each KV head, in token-major or head-major order,
// at any element strides with contiguous channels -- repacks it once with
// lbsr_pack_cache, and can read it back with lbsr_unpack_cache.
//
// One workgroup per (page, KV head) tile.  The tile is read with 16-byte loads
// into LDS in its source order, rearranged element by element inside LDS with
// the same element offsets the prologue's cache write uses, and written out
// with 16-byte stores, so both HBM streams stay coalesced.  FP8 codes are
// bytes moved as they are: no scale is applied.

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace lbsr {

constexpr int kPackThreads = 256;

template <bool kFp8, bool kV>
__device__ __forceinline__ int tile_offset(int r, int d) {
  if constexpr (kFp8) return kV ? v_offset_fp8(r, d) : k_offset_fp8(r, d);
  else return kV ? v_offset_bf16(r, d) : k_offset_bf16(r, d);
}

// kPack: rows -> tile; else tile -> rows.  Strides in elements of the cache
// dtype; the host has checked alignment and that no two rows overlap.
template <bool kFp8, bool kV, bool kPack>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(
    const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t tile_page_stride,
    int64_t tile_head_stride, int64_t row_page_stride, int64_t row_token_stride,
    int64_t row_head_stride) {
  using Elem = typename std::conditional<kFp8, uint8_t, uint16_t>::type;
  constexpr int kElem = sizeof(Elem);
  constexpr int kChunks = kTileElems * kElem / 16;          // 16-byte pieces of a tile
  constexpr int kChunksPerRow = kHeadDim * kElem / 16;      // of one token row
  __shared__ u32x4 s_in[kChunks];
  __shared__ u32x4 s_out[kChunks];

  const int64_t page = blockIdx.x;
  const int64_t g = blockIdx.y;
  const int tid = threadIdx.x;
  const size_t tile_base = (size_t)(page * tile_page_stride + g * tile_head_stride) * kElem;
  const size_t row_base = (size_t)(page * row_page_stride + g * row_head_stride) * kElem;
  const size_t row_step = (size_t)row_token_stride * kElem;
  // 16-byte piece c of the tile as rows: row c / kChunksPerRow, channels from
  // (c % kChunksPerRow) * 16 / kElem
  auto row_piece = [&](uint8_t* base, int c) {
    return (u32x4*)(base + row_base + (size_t)(c / kChunksPerRow) * row_step +
                    (size_t)(c % kChunksPerRow) * 16);
  };

#pragma unroll
  for (int i = 0; i < kChunks / kPackThreads; ++i) {
    const int c = tid + i * kPackThreads;
    s_in[c] = kPack ? *row_piece(const_cast<uint8_t*>(src), c)
                    : *(const u32x4*)(src + tile_base + (size_t)c * 16);
  }
  __syncthreads();
  // element (row r, channel d): position r * 128 + d in row order, the tile
  // offset in tile order
  const Elem* in = (const Elem*)s_in;
  Elem* out = (Elem*)s_out;
  for (int i = tid; i < kTileElems; i += kPackThreads) {
    const int r = i >> 7, d = i & (kHeadDim - 1);
    const int o = tile_offset<kFp8, kV>(r, d);
    if constexpr (kPack) out[o] = in[i];
    else out[i] = in[o];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kChunks / kPackThreads; ++i) {
    const int c = tid + i * kPackThreads;
    if constexpr (kPack) *(u32x4*)(dst + tile_base + (size_t)c * 16) = s_out[c];
    else *row_piece(dst, c) = s_out[c];
  }
}

hipError_t launch_pack(bool fp8, bool v, bool pack, const void* src, void* dst, int64_t num_pages,
                       int num_kv_heads, int64_t tile_page_stride, int64_t tile_head_stride,
                       int64_t row_page_stride, int64_t row_token_stride, int64_t row_head_stride,
                       hipStream_t stream) {
  const dim3 grid((unsigned)num_pages, (unsigned)num_kv_heads);
  auto go = [&](auto kernel) {
    kernel<<<grid, kPackThreads, 0, stream>>>((const uint8_t*)src, (uint8_t*)dst,
                                              tile_page_stride, tile_head_stride, row_page_stride,
                                              row_token_stride, row_head_stride);
  };
  auto by_dir = [&](auto f8, auto vv) {
    constexpr bool F = decltype(f8)::value, V = decltype(vv)::value;
    if (pack) go(pack_kernel<F, V, true>);
    else go(pack_kernel<F, V, false>);
  };
  auto by_kind = [&](auto f8) {
    if (v) by_dir(f8, std::true_type{});
    else by_dir(f8, std::false_type{});
  };
  if (fp8) by_kind(std::true_type{});
  else by_kind(std::false_type{});
  return hipGetLastError();
}

}  // namespace lbsr
