// Per-step tile schedule, computed on the device in one workgroup.
//
// [A] "Why does dynamic scheduling matter in attention?": tiles of 64 tokens
// are dealt to the compute units in proportion to each sequence's current
// length, every step, instead of a static split-KV that assumes equal
// lengths.  Reading of "proportional": all tiles of the batch are laid end to
// end (T in total) and worker w of P takes flat tiles
// [floor(w*T/P), floor((w+1)*T/P)), so loads differ by at most one tile; a
// worker's range is cut at sequence ends into chunks.  The static baseline
// cuts every sequence into the same S parts of its own length.
//
// Weighted variant (an MI355X refinement; equal weights give the rule above
// exactly): MI355X's XCDs stream HBM at different rates (about 10% apart
// between the fastest and slowest under a full-chip stream), so equal shares
// leave the fast XCDs idle at the end.  With per-XCD weights, worker w takes
// [floor(T*C(w)/C(P)), floor(T*C(w+1)/C(P))) where C(w) sums the weights of
// workers 0..w-1 and a worker weighs the weight of the XCD that runs it.
//
// One 1024-thread workgroup: per-sequence prefix sums live in LDS (s_cu holds
// batch + 1 ints, batch <= 16384); counts per worker are scanned in
// 1024-wide rounds with a carry.
// Everything is integer arithmetic; products T*C(w) are 64-bit.

#pragma once

#include "common.h"

namespace lbsr {

// Inclusive block scan of one int per thread (1024 threads = 16 waves): a
// shuffle scan inside each wave, then wave 0 scans the 16 wave totals.
__device__ inline int block_inclusive_scan(int x, int* s_wave, int& total) {
  constexpr int kWaves = kPlanThreads / kWave;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int t = lane < kWaves ? s_wave[lane] : 0;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const int y = __shfl_up(t, d, kWave);
      if (lane >= d) t += y;
    }
    if (lane < kWaves) s_wave[lane + 1] = t;  // inclusive totals, shifted: exclusive offsets
    if (lane == 0) s_wave[0] = 0;
  }
  __syncthreads();
  x += s_wave[wave];
  total = s_wave[kWaves];
  __syncthreads();  // s_wave is reused by the next call
  return x;
}

// Index of the sequence that holds flat tile t: the largest b with cu[b] <= t.
__device__ inline int seq_of_tile(const int* cu, int batch, int t) {
  int lo = 0, hi = batch;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// C(w): summed weight of workers 0..w-1 (w itself when unweighted).  XCD x
// runs the contiguous workers that follow XCD x-1's.
__device__ inline int64_t cumulative_weight(const SchedParams& sp, int w) {
  if (!sp.weighted) return w;
  int64_t c = 0;
  int start = 0;
  for (int x = 0; x < kXcds; ++x) {
    const int n = xcd_run_size(x, sp.num_workers);
    if (w < start + n) return c + (int64_t)(w - start) * sp.xcd_weight[x];
    c += (int64_t)n * sp.xcd_weight[x];
    start += n;
  }
  return c;
}

// The whole schedule, computed by one 1024-thread workgroup; s_cu is LDS of
// at least batch + 1 ints.
__device__ inline void plan_body(const int32_t* __restrict__ seq_lens, int batch, int max_blocks,
                                 const SchedParams& sp, const PlanPtrs& plan, int* s_cu) {
  const int dynamic = sp.dynamic, num_workers = sp.num_workers, splits = sp.splits;
  __shared__ int s_wave[kPlanThreads / kWave + 1];
  const int tid = threadIdx.x;
  if (tid == 0) plan.error_word[0] = 0;

  // 1. clamped lengths, tiles per sequence, prefix sums
  const int max_len = max_blocks * kPage;
  int bad = 0;
  int carry = 0;
  if (tid == 0) s_cu[0] = 0;
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int b = base + tid;
    int n = 0;
    if (b < batch) {
      const int L = seq_lens[b];
      const int Lc = L < sp.min_len ? sp.min_len : (L > max_len ? max_len : L);
      bad |= (Lc != L);
      plan.seq_len_eff[b] = Lc;
      n = (Lc + kPage - 1) / kPage;
    }
    int total;
    const int incl = block_inclusive_scan(n, s_wave, total);
    if (b < batch) s_cu[b + 1] = carry + incl;
    carry += total;
  }
  if (bad) atomicOr(plan.error_word, (int32_t)kErrSeqLen);
  __syncthreads();
  for (int b = tid; b <= batch; b += kPlanThreads) plan.cu_tiles[b] = s_cu[b];
  const int T = s_cu[batch];

  // 2. chunk counts per worker, their prefix sums, and the chunks themselves
  const int W = dynamic ? num_workers : batch * splits;
  const int64_t c_total = dynamic ? cumulative_weight(sp, W) : 1;  // <= 1024 * 65536
  carry = 0;
  for (int base = 0; base < W; base += kPlanThreads) {
    const int w = base + tid;
    int cnt = 0, first = 0;
    int s = 0, e = 0;
    if (w < W) {
      if (dynamic) {
        // T < 2^31 and C(w) <= 2^26: the products fit in 64 bits
        s = (int)(((int64_t)T * cumulative_weight(sp, w)) / c_total);
        e = (int)(((int64_t)T * cumulative_weight(sp, w + 1)) / c_total);
        if (s < e) {
          first = seq_of_tile(s_cu, batch, s);
          cnt = seq_of_tile(s_cu, batch, e - 1) - first + 1;
        }
      } else {
        const int b = w / splits, part = w - b * splits;
        const int n = s_cu[b + 1] - s_cu[b];
        s = (int)(((int64_t)part * n) / splits);
        e = (int)(((int64_t)(part + 1) * n) / splits);
        first = b;
        cnt = e > s ? 1 : 0;
      }
    }
    int total;
    const int c0 = carry + block_inclusive_scan(cnt, s_wave, total) - cnt;
    if (w < W) {
      plan.worker_chunk[w] = c0;
      for (int i = 0; i < cnt; ++i) {
        const int c = c0 + i;
        const int b = first + i;
        int t0, t1;
        if (dynamic) {
          const int a = s > s_cu[b] ? s : s_cu[b];
          const int z = e < s_cu[b + 1] ? e : s_cu[b + 1];
          t0 = a - s_cu[b];
          t1 = z - s_cu[b];
        } else {
          t0 = s;
          t1 = e;
        }
        int32_t* ch = plan.chunks + 4 * (size_t)c;
        ch[0] = b;
        ch[1] = t0;
        ch[2] = t1;
        ch[3] = w;
        if (t0 == 0) plan.seq_chunk[b] = c;  // a sequence's first chunk starts at its tile 0
      }
    }
    carry += total;
  }
  if (tid == 0) {
    plan.worker_chunk[W] = carry;
    plan.seq_chunk[batch] = carry;
  }
  // the folded merge's arrival counters start from zero every step
  for (int i = tid; i < batch * sp.fold_groups; i += kPlanThreads) plan.arrivals[i] = 0;
}


}  // namespace lbsr
