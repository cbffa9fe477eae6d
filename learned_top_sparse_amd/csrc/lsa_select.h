// lsa_select.h -- pieces of the exact top-k selection shared by the selection
// kernels and the indexer that can build a row's score histogram as it goes.
#pragma once
#include "lsa_device.h"
#include "lsa_internal.h"

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

// The same layout for 64-bit scores with 6 mantissa bits: u = s folded (s ^ sign),
// shift = max(0, 57 - clz(u)), g = (shift << 6) + (u >> shift) < 3712 (u itself below 128,
// 64 bins per power of two above), bin = 4096 + g for s >= 0 and 4095 - g below.
__device__ __forceinline__ int coarse_bin64(long long s) {
  const long long sign = s >> 63;
  const unsigned long long u = (unsigned long long)(s ^ sign);
  const int shift = max(0, 57 - (int)__clzll((long long)(u | 1ull)));
  const int gv = (shift << 6) + (int)(u >> shift);
  return (gv ^ (int)sign) + 4096;
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

constexpr int INFO = 8;
constexpr int GRP = 32;
constexpr int NGRP = NBINS / GRP;
// slots per workgroup in the several-workgroups-per-row top-k
constexpr int SEG = 8192;

// Smallest score whose coarse bin is >= bw (bins 896..7295 are the ones coarse_bin
// produces): coarse_bin(s) >= bw  <=>  s >= bin_floor(bw).  Inverts the mapping above:
// g values below 256 are u itself; g >= 256 has shift g/128 - 1 and mantissa
// 128 + g%128.  On the negative side the bin of ~u falls as u grows, so the bound is
// -(smallest u of the next g value).
__device__ __forceinline__ int bin_floor(int bw) {
  auto umin_of = [](int gv) -> unsigned {
    return gv < 256 ? (unsigned)gv : (unsigned)(128 + (gv & 127)) << ((gv >> 7) - 1);
  };
  if (bw >= 4096) return (int)umin_of(bw - 4096);
  const int g1 = 4096 - bw;
  return g1 > 3199 ? INT_MIN : -(int)umin_of(g1);
}

// Decode selection (flat rows, the indexer builds the selection state): every row's
// n_valid keys are cut into `parts` spans of dec_span(n_valid, parts) consecutive keys,
// one indexer workgroup each.  A span's scores stay in that workgroup's LDS, so a span
// holds at most DEC_SPAN_MAX keys; the launch aims at DEC_WGS workgroups (one per
// compute unit of an MI355X) with spans of at least DEC_SPAN_MIN keys.
constexpr int DEC_SPAN_MAX = 34816;
constexpr int DEC_WGS = 256;
constexpr int DEC_SPAN_MIN = 2048;
constexpr int DEC_MAX_PARTS = 1024;  // the per-row finish takes one span per thread
__host__ __device__ __forceinline__ int dec_span(int n_valid, int parts) {
  return ((n_valid + parts - 1) / parts + 63) / 64 * 64;
}

// What each decode-indexer workgroup leaves for the per-row finish, one record per
// (row, span), written in full with plain stores (nothing to clear beforehand):
//   hdr[4] = {lo, hi, lcnt, lbw}: the band of coarse bins its scores fall in, its
//     list length and the lowest bin its list takes (-1: no list, its scores are in
//     its slice of the score table);
//   gsum[NGRP]: its counts per group of GRP bins;
//   hist[NBINS]: its counts per bin, bins lo..hi only;
//   lslot[lcap], lscore[lcap]: the list's slots and scores, in slot order (lcap is a
//     multiple of 4, so both arrays are 16-byte aligned and a reader may take them a
//     quad at a time up to the count rounded up to 4).
// Records of one row are consecutive; rows are `parts` records apart.
struct DecWs {
  int* base;
  long long rec_ints;
  int parts, lcap;
  __host__ __device__ static constexpr long long rec_ints_for(long long lcap) {
    return (4 + NGRP + NBINS + 2 * lcap + 3) / 4 * 4;
  }
  __device__ __forceinline__ int* rec(long long row, int p) const { return base + (row * parts + p) * rec_ints; }
  __device__ __forceinline__ int* hdr(long long row, int p) const { return rec(row, p); }
  __device__ __forceinline__ int* gsum(long long row, int p) const { return rec(row, p) + 4; }
  __device__ __forceinline__ int* hist(long long row, int p) const { return rec(row, p) + 4 + NGRP; }
  __device__ __forceinline__ int* lslot(long long row, int p) const { return rec(row, p) + 4 + NGRP + NBINS; }
  __device__ __forceinline__ int* lscore(long long row, int p) const { return lslot(row, p) + lcap; }
};

// Per-row selection state of the several-workgroups top-k in its workspace (rows
// row_ints_for(n_seg) ints apart, a multiple of 4, so every row's histogram is
// 16-byte aligned):
//   hist[NBINS] | info[INFO] = {b*, above, cnt*, overflow, arrivals, -, -, -} |
//   gsum[NGRP] (unused here) | cnt[n_seg] | cand[n_seg][CAP] (slot, score) pairs
struct SegWs {
  int* base;
  int n_seg;
  __host__ __device__ static constexpr long long row_ints_for(long long n_seg) {
    return (NBINS + INFO + NGRP + n_seg + 2 * n_seg * CAP + 3) / 4 * 4;
  }
  __host__ __device__ long long row_ints() const { return row_ints_for(n_seg); }
  __device__ __forceinline__ int* hist(long long r) const { return base + r * row_ints(); }
  __device__ __forceinline__ int* info(long long r) const { return hist(r) + NBINS; }
  __device__ __forceinline__ int* gsum(long long r) const { return info(r) + INFO; }
  __device__ __forceinline__ int* cnt(long long r) const { return gsum(r) + NGRP; }
  __device__ __forceinline__ int* cand(long long r, int seg) const { return cnt(r) + n_seg + 2ll * seg * CAP; }
};

// Ordered compaction over positions [0, n): pred(pos, payload&) selects; emit(rank,
// pos, payload) is called for selected positions with their rank in position order.
// wcnt: LDS int[2 * V * NT/64].  All threads must call; returns the count.
template <int NT, int V, typename Pred, typename Emit>
__device__ __forceinline__ int ordered_compact(int n, int* wcnt, Pred pred, Emit emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int running = 0, parity = 0;
  for (int base = 0; base < n; base += V * NT) {
    bool f[V];
    int pl[V];
    unsigned long long bal[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int pos = base + v * NT + (int)threadIdx.x;
      pl[v] = 0;
      f[v] = (pos < n) && pred(pos, pl[v]);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) bal[v] = __ballot(f[v]);
    int* wc = wcnt + parity * V * NW;
    if (lane == 0) {
#pragma unroll
      for (int v = 0; v < V; ++v) wc[v * NW + wave] = __popcll(bal[v]);
    }
    __syncthreads();
    int off = running;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      int pre = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = wc[v * NW + w];
        pre += (w < wave) ? c : 0;
        tot += c;
      }
      if (f[v]) emit(off + pre + lanes_below(bal[v]), base + v * NT + (int)threadIdx.x, pl[v]);
      off += tot;
    }
    running = off;
    parity ^= 1;
  }
  __syncthreads();
  return running;
}



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

// ---------------------------------------------------------------------------------
// Exact selection over 64-bit keys held in registers, C <= 32 per thread: key c of thread
// t sits at position c * NT + t and counts iff bit c of vmask is set.  All threads call.

// The need-th largest of the valid keys (1 <= need <= their number): radix passes of
// 11-bit digits below the prefix shared by the largest and smallest valid key, counted
// in an LDS histogram (hist: 2048 ints).  Returns T; *need_eq = how many keys equal to
// T are among the need largest.
template <int NT, int C>
__device__ __forceinline__ unsigned long long radix_cut64(const unsigned long long (&key)[C], unsigned vmask,
                                                          int need, int* hist, int* scan_tmp, int* sh,
                                                          unsigned long long* shu, int* need_eq) {
  static_assert(C <= 32, "a 32-bit validity mask");
  constexpr int DIG = 11, NBIN = 1 << DIG;
  constexpr int BPT = (NBIN + NT - 1) / NT;  // bins per thread in the scan
  const int tid = threadIdx.x, lane = tid & 63;
  unsigned long long mx = 0ull, mn = ~0ull;
#pragma unroll
  for (int c = 0; c < C; ++c)
    if ((vmask >> c) & 1u) {
      mx = key[c] > mx ? key[c] : mx;
      mn = key[c] < mn ? key[c] : mn;
    }
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long a = __shfl_xor(mx, o), b = __shfl_xor(mn, o);
    mx = a > mx ? a : mx;
    mn = b < mn ? b : mn;
  }
  if (tid == 0) {
    shu[0] = 0ull;
    shu[1] = ~0ull;
  }
  __syncthreads();
  if (lane == 0) {
    atomicMax(&shu[0], mx);
    atomicMin(&shu[1], mn);
  }
  __syncthreads();
  mx = shu[0];
  mn = shu[1];
  unsigned long long pref = mx, pmask = ~0ull;
  if (mx != mn) {
    const int hb = 63 - __clzll((long long)(mx ^ mn));  // highest bit where keys differ
    pmask = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
    pref = mx & pmask;
    for (int top = hb; top >= 0; top -= DIG) {
      const int lo = max(0, top - DIG + 1);
      const int nb = 1 << (top - lo + 1);
      for (int t = tid; t < nb; t += NT) hist[t] = 0;
      __syncthreads();
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (((vmask >> c) & 1u) && (key[c] & pmask) == pref) atomicAdd(&hist[(int)((key[c] >> lo) & (nb - 1))], 1);
      __syncthreads();
      // thread t sums bins nb-1-BPT*t .. nb-BPT*(t+1) (from the top); the one whose range
      // holds the need-th entry walks it
      int csum = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        const int bin = nb - 1 - BPT * tid - j;
        csum += bin >= 0 ? hist[bin] : 0;
      }
      int tot;
      const int excl = block_exclusive_scan<NT>(csum, scan_tmp, &tot);
      if (excl < need && excl + csum >= need) {
        int acc = excl;
        for (int j = 0; j < BPT && nb - 1 - BPT * tid - j >= 0; ++j) {
          const int bin = nb - 1 - BPT * tid - j;
          const int h = hist[bin];
          if (acc + h >= need) {
            sh[0] = bin;
            sh[1] = acc;
            break;
          }
          acc += h;
        }
      }
      __syncthreads();
      need -= sh[1];
      pref |= (unsigned long long)sh[0] << lo;
      pmask |= (unsigned long long)(nb - 1) << lo;
      __syncthreads();
    }
  }
  *need_eq = need;
  return pref;
}

// Adds to the LDS bitmap bm the need_eq lowest positions set in eqm (nwd words each):
// the keys equal to the cut that the keep takes.  All threads call, with eqm complete;
// bm is complete when this returns.
template <int NT>
__device__ __forceinline__ void keep_first_ties(unsigned* bm, const unsigned* eqm, int nwd, int need_eq,
                                                int* scan_tmp) {
  const int tid = threadIdx.x;
  // each thread takes whole words in order: the rank of its first equal key among all
  const int wpt = (nwd + NT - 1) / NT;
  int n_eq = 0;
  for (int j = 0; j < wpt; ++j) {
    const int wd = wpt * tid + j;
    if (wd < nwd) n_eq += __popc(eqm[wd]);
  }
  int tot;
  int before = block_exclusive_scan<NT>(n_eq, scan_tmp, &tot);
  for (int j = 0; j < wpt; ++j) {
    const int wd = wpt * tid + j;
    if (wd >= nwd) break;
    unsigned e = eqm[wd], keep = 0u;
    while (e != 0u && before < need_eq) {
      const unsigned low = e & (0u - e);
      keep |= low;
      e ^= low;
      ++before;
    }
    bm[wd] |= keep;
  }
  __syncthreads();
}

// Marks, in an LDS bitmap of positions (bm: NT * C / 32 words), the keys kept by the cut:
// key > T, and the first need_eq keys equal to T in position order (the lowest
// positions win ties).  eqm: another NT * C / 32 words of LDS.  The bitmap is complete
// when this returns.
template <int NT, int C>
__device__ __forceinline__ void mark_kept64(const unsigned long long (&key)[C], unsigned vmask,
                                            unsigned long long T, int need_eq, unsigned* bm, unsigned* eqm,
                                            int* scan_tmp) {
  constexpr int NWD = NT * C / 32;
  static_assert(NT * C % 32 == 0, "whole bitmap words");
  const int tid = threadIdx.x;
  __syncthreads();
  for (int t = tid; t < NWD; t += NT) {
    bm[t] = 0u;
    eqm[t] = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < C; ++c) {
    if (!((vmask >> c) & 1u)) continue;
    const int pos = c * NT + tid;
    if (key[c] > T) atomicOr(&bm[pos >> 5], 1u << (pos & 31));
    else if (key[c] == T) atomicOr(&eqm[pos >> 5], 1u << (pos & 31));
  }
  __syncthreads();
  keep_first_ties<NT>(bm, eqm, NWD, need_eq, scan_tmp);
}

// Writes the marked positions in ascending order: emit(rank, pos) for each; returns
// their number.  Each thread takes whole words of the bitmap (NWD words).
template <int NT, typename Emit>
__device__ __forceinline__ int emit_marked(const unsigned* bm, int NWD, int* scan_tmp, Emit emit) {
  const int tid = threadIdx.x;
  const int WPT = (NWD + NT - 1) / NT;
  int mine = 0;
  for (int j = 0; j < WPT; ++j) {
    const int wd = WPT * tid + j;
    if (wd < NWD) mine += __popc(bm[wd]);
  }
  int tot;
  int r = block_exclusive_scan<NT>(mine, scan_tmp, &tot);
  for (int j = 0; j < WPT; ++j) {
    const int wd = WPT * tid + j;
    if (wd >= NWD) break;
    unsigned bits = bm[wd];
    while (bits != 0u) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1u;
      emit(r, 32 * wd + bit);
      ++r;
    }
  }
  return tot;
}

}  // namespace lsa
