// lsa_select.h -- pieces of the exact top-k selection shared by the selection
// kernels and the indexer that can build a row's score histogram as it goes.
#pragma once
#include "lsa_device.h"

namespace lsa {

constexpr int NBINS = 8192;
constexpr int CAP = NBINS / 2;  // LDS list entries (slot, score), reusing the histogram storage

// Monotone 13-bit bin: non-negative scores map to 4096 + g(s), negative ones to
// 4095 - g(~s), where g keeps the exponent and the top 7 mantissa bits:
//   u = |s| folded (s ^ sign), shift = max(0, 24 - clz(u)), g = (shift << 7) + (u >> shift).
// For u < 128 this is u itself; above, each power of two is split into 128 bins.
__device__ __forceinline__ int coarse_bin(int s) {
  const int sign = s >> 31;
  const unsigned u = (unsigned)(s ^ sign);
  const int shift = max(0, 24 - (int)__clz((int)(u | 1u)));
  const int gv = (shift << 7) + (int)(u >> shift);
  return (gv ^ sign) + 4096;
}

// Bin b* holding the k-th best entry of `hist` (NBINS counters, LDS or global):
// writes sh[4] = b*, sh[5] = entries in bins above b*, sh[6] = entries in b*.
template <int NT>
__device__ __forceinline__ void find_cut_bin(const int* hist, int k, int* scan_tmp, int* sh) {
  constexpr int C = NBINS / NT;
  const int hi = NBINS - (int)threadIdx.x * C;
  int csum = 0;
  // skewed visiting order: at step i lane t reads bin (i + t) % C of its range, so the
  // lanes of a wave touch distinct LDS banks
#pragma unroll 8
  for (int i = 0; i < C; ++i) csum += hist[hi - C + ((i + (int)threadIdx.x) & (C - 1))];
  int tot;
  const int excl = block_exclusive_scan<NT>(csum, scan_tmp, &tot);
  if (excl < k && excl + csum >= k) {
    int acc = excl;
    for (int b = hi - 1; b >= hi - C; --b) {
      const int h = hist[b];
      if (acc + h >= k) {
        sh[4] = b;
        sh[5] = acc;
        sh[6] = h;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

// Per-row selection state kept in device memory between the kernels of a row:
//   hist[NBINS] | info[8] = {b*, above, cnt*, overflow, arrivals, -, -, -} |
//   gsum[NGRP] (sums of GRP consecutive bins; kept only where the indexer builds
//   the histogram) | ...
constexpr int INFO = 8;
constexpr int GRP = 32;
constexpr int NGRP = NBINS / GRP;

// Adds a workgroup's LDS histogram `hist` (NBINS counters, complete when called) into
// the row's device histogram `gh`.  The last of the row's `n_parts` workgroups to
// arrive finds the cut bin for everyone and writes info[0..3].  Each workgroup
// waits for its own histogram atomics to be performed (s_waitcnt, no cache
// write-back fence) before it counts itself in; the last one reads the totals back
// with device-scope atomic loads.  `hist` is overwritten by the last workgroup.
template <int NT>
__device__ __forceinline__ void merge_row_histogram(int* hist, int* gh, int* info, int n_parts, int k,
                                                    int* scan_tmp, int* sh) {
  for (int t = threadIdx.x; t < NBINS; t += NT) {
    const int h = hist[t];
    if (h) atomicAdd(&gh[t], h);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) sh[7] = (atomicAdd(&info[4], 1) == n_parts - 1);
  __syncthreads();
  if (!sh[7]) return;
  for (int t = threadIdx.x; t < NBINS; t += NT)
    hist[t] = __hip_atomic_load(&gh[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  find_cut_bin<NT>(hist, k, scan_tmp, sh);
  if (threadIdx.x == 0) {
    info[0] = sh[4];
    info[1] = sh[5];
    info[2] = sh[6];
    info[3] = (sh[5] + sh[6] > CAP) ? 1 : 0;
  }
}

}  // namespace lsa
