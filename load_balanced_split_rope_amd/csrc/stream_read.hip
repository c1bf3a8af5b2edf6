// A streaming-read probe: the measured HBM ceiling that the split-attention
// kernel's bandwidth is compared against.  It reads device memory the way the
// split kernel reads K/V tiles -- non-temporal 16-byte loads, one 32 KiB
// burst per wave (32 fragments of 1 KiB, as one BF16 tile's K and V), eight
// waves per workgroup, one workgroup per compute unit by default -- and does
// nothing with the bytes except fold them into a checksum, so the compiler
// keeps every load.

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
  uint32_t acc = 0;
  for (int64_t blk = (int64_t)blockIdx.x * kProbeWaves + wave; blk < blocks; blk += stride) {
    const u32x4* p = buf + blk * (kProbeFrags * kWave);
    u32x4 r[kProbeFrags];
#pragma unroll
    for (int f = 0; f < kProbeFrags; ++f) r[f] = __builtin_nontemporal_load(p + f * kWave + lane);
#pragma unroll
    for (int f = 0; f < kProbeFrags; ++f) acc ^= r[f].x ^ r[f].y ^ r[f].z ^ r[f].w;
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

hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                              hipStream_t stream) {
  const int64_t blocks = (int64_t)(bytes / kProbeBlockBytes);
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kProbeWaves * kWave), 0, stream,
                     (const u32x4*)buf, blocks, sink);
  return hipGetLastError();
}

}  // namespace lbsr
