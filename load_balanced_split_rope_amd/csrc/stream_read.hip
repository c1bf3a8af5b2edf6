// A streaming-read probe: the measured HBM ceiling that the split-attention
// kernel's bandwidth is compared against.  Form 0 reads device memory the way the
// split kernel reads K/V tiles -- non-temporal 16-byte loads, one 32 KiB
// burst per wave (32 fragments of 1 KiB, as one BF16 tile's K and V), eight
// waves per workgroup in lockstep (a workgroup barrier after each burst is
// issued), one workgroup per compute unit by default -- and does
// nothing with the bytes except fold them into a checksum, so the compiler
// keeps every load.  Form 1 is a plain grid-wide sweep (below).  Form 2 is
// form 0 with the bytes going straight into LDS by global-to-LDS loads
// (16 KiB bursts: 8 waves x 16 KiB fill 128 KiB of LDS), read back from LDS
// into the checksum.

#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"

namespace lbsr {

namespace {

constexpr int kProbeWaves = 8;
constexpr int kProbeFrags = 32;                     // 1 KiB fragments per burst
constexpr int64_t kProbeBlockBytes = kProbeFrags * 1024;

__global__ __launch_bounds__(kProbeWaves * kWave) void stream_read_kernel(
    const u32x4* __restrict__ buf, int64_t blocks, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int64_t stride = (int64_t)gridDim.x * kProbeWaves;
  // every wave of a workgroup makes the same number of passes (a block past
  // the end is skipped, its barrier still taken), so the barrier below is
  // reached by all of them each pass
  const int64_t passes = (blocks + stride - 1) / stride;
  uint32_t acc = 0;
  for (int64_t it = 0; it < passes; ++it) {
    const int64_t blk = it * stride + (int64_t)blockIdx.x * kProbeWaves + wave;
    const bool live = blk < blocks;
    const u32x4* p = buf + (live ? blk : 0) * (kProbeFrags * kWave);
    u32x4 r[kProbeFrags];
    if (live) {
#pragma unroll
      for (int f = 0; f < kProbeFrags; ++f) r[f] = __builtin_nontemporal_load(p + f * kWave + lane);
    }
    // waves in lockstep, the loads still in flight (as the split kernel's waves)
    __builtin_amdgcn_s_barrier();
    if (live) {
#pragma unroll
      for (int f = 0; f < kProbeFrags; ++f) acc ^= r[f].x ^ r[f].y ^ r[f].z ^ r[f].w;
    }
  }
  for (int d = 1; d < kWave; d <<= 1) acc ^= __shfl_xor(acc, d, kWave);
  __shared__ uint32_t s_acc[kProbeWaves];
  if (lane == 0) s_acc[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kProbeWaves; ++w) x ^= s_acc[w];
    sink[blockIdx.x] = x;
  }
}

// The plain form: no bursts, no barriers.  Each pass, every thread keeps
// kProbeDepth 16-byte loads in flight, one grid-width apart, so the whole grid
// sweeps the buffer front to back.
constexpr int kProbeDepth = 8;

__global__ __launch_bounds__(kProbeWaves * kWave) void stream_read_plain_kernel(
    const u32x4* __restrict__ buf, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t width = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (int64_t base = 0; base < n16; base += kProbeDepth * width) {
    u32x4 r[kProbeDepth];
#pragma unroll
    for (int k = 0; k < kProbeDepth; ++k) {
      const int64_t i = base + k * width + tid;
      r[k] = i < n16 ? __builtin_nontemporal_load(buf + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < kProbeDepth; ++k) acc ^= r[k].x ^ r[k].y ^ r[k].z ^ r[k].w;
  }
  for (int d = 1; d < kWave; d <<= 1) acc ^= __shfl_xor(acc, d, kWave);
  __shared__ uint32_t s_acc[kProbeWaves];
  if ((threadIdx.x % kWave) == 0) s_acc[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kProbeWaves; ++w) x ^= s_acc[w];
    sink[blockIdx.x] = x;
  }
}

// Form 2: each wave's 16 KiB burst lands in its own 16 KiB of LDS; the waves
// meet at a barrier with the loads in flight, then each waits for its own and
// folds its LDS slice into the checksum.
constexpr int kLdsFrags = 16;

__global__ __launch_bounds__(kProbeWaves * kWave) void stream_read_lds_kernel(
    const u32x4* __restrict__ buf, int64_t blocks, uint32_t* __restrict__ sink) {
  __shared__ u32x4 s_buf[kProbeWaves * kLdsFrags * kWave];   // 128 KiB
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  u32x4* mine = s_buf + wave * kLdsFrags * kWave;
  const int64_t stride = (int64_t)gridDim.x * kProbeWaves;
  const int64_t passes = (blocks + stride - 1) / stride;
  uint32_t acc = 0;
  for (int64_t it = 0; it < passes; ++it) {
    const int64_t blk = it * stride + (int64_t)blockIdx.x * kProbeWaves + wave;
    const bool live = blk < blocks;
    const u32x4* p = buf + (live ? blk : 0) * (kLdsFrags * kWave);
    if (live) {
#pragma unroll
      for (int f = 0; f < kLdsFrags; ++f)
        __builtin_amdgcn_global_load_lds((const void*)(p + f * kWave + lane),
                                         (__attribute__((address_space(3))) void*)(mine + f * kWave),
                                         16, 0, 2);
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's slice is in LDS
    if (live) {
#pragma unroll
      for (int f = 0; f < kLdsFrags; ++f) {
        const u32x4 r = mine[f * kWave + lane];
        acc ^= r.x ^ r.y ^ r.z ^ r.w;
      }
    }
  }
  for (int d = 1; d < kWave; d <<= 1) acc ^= __shfl_xor(acc, d, kWave);
  __shared__ uint32_t s_acc[kProbeWaves];
  if (lane == 0) s_acc[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kProbeWaves; ++w) x ^= s_acc[w];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

int64_t stream_read_block_bytes() { return kProbeBlockBytes; }

hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, int mode,
                              uint32_t* sink, hipStream_t stream) {
  if (mode == 0) {
    const int64_t blocks = (int64_t)(bytes / kProbeBlockBytes);
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kProbeWaves * kWave), 0,
                       stream, (const u32x4*)buf, blocks, sink);
  } else if (mode == 2) {
    const int64_t blocks = (int64_t)(bytes / (kLdsFrags * 1024));
    hipLaunchKernelGGL(stream_read_lds_kernel, dim3(workgroups), dim3(kProbeWaves * kWave), 0,
                       stream, (const u32x4*)buf, blocks, sink);
  } else {
    hipLaunchKernelGGL(stream_read_plain_kernel, dim3(workgroups), dim3(kProbeWaves * kWave), 0,
                       stream, (const u32x4*)buf, (int64_t)(bytes / 16), sink);
  }
  return hipGetLastError();
}

}  // namespace lbsr
