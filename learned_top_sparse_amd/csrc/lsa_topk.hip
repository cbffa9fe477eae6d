// lsa_topk.hip -- exact per-query top-k with lowest-index tie-break (gfx950).
//
// Semantics (HyScale summary: HyTopK computes each query's exact top-k; "Latent
// Sparse Attention (LSA)" App. F.1 "Selection by threshold": a better score ranks
// first and, at equal score, the lower id; "Attention kernels": the list is a row
// of int32 padded with -1).  The output row lists the selected keys in ascending
// key order, which is what a stable, order-preserving compaction yields for free.
//
// One workgroup per query row.  The cut is found the way the LSA page's expansion
// does it, by radix select over integer keys, but with a first digit adapted to
// indexer scores: a 13-bit monotone "sign / exponent / 7 mantissa bits" bin, so one
// histogram pass over the row isolates a bin holding only a few hundred entries
// for smooth score distributions.
//   1. histogram of the coarse bin over the row (LDS atomics);
//   2. find the bin b* holding the k-th best entry (block scan from the top);
//   3. stable compaction of every entry in bins >= b* into an LDS list, in slot
//      order (wave ballots + one barrier per 16*NT entries);
//   4. exact 8-bit radix passes over the b* entries only, giving the threshold
//      score T and how many entries equal to T to take (lowest slots first);
//   5. stable compaction of the list into the output row.
// If bins >= b* hold more than the LDS list can take (heavy ties, adversarial
// distributions), the row falls back to exact 8-bit radix passes and a final
// stable compaction over the row in global memory.  Every path is exact.
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

namespace {

constexpr int NBINS = 8192;
constexpr int CAP = NBINS / 2;  // LDS list entries (slot, score), reusing the histogram storage

__device__ __forceinline__ unsigned okey(int s) { return (unsigned)s ^ 0x80000000u; }

// Monotone 13-bit bin: non-negative scores map to 4096 + g(s), negative ones to
// 4095 - g(~s), where g keeps the exponent and the top 7 mantissa bits.
__device__ __forceinline__ int coarse_bin(int s) {
  const unsigned u = s >= 0 ? (unsigned)s : ~(unsigned)s;
  int gv;
  if (u < 128u) {
    gv = (int)u;
  } else {
    const int e = 31 - __clz((int)u);
    gv = ((e - 6) << 7) + (int)((u >> (e - 7)) & 127u);
  }
  return s >= 0 ? 4096 + gv : 4095 - gv;
}

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

// Among positions [0, n) accepted by pred (payload = score), find the need-th best
// score by 8-bit radix passes on the order-preserving key.  Returns T (as key) and
// sets *need_eq to how many entries equal to T are selected.  All threads call.
template <int NT, int V, typename Pred>
__device__ __forceinline__ unsigned radix_select32(int n, int need, int* h256, int* scan_tmp, int* sh,
                                                   Pred pred, int* need_eq) {
  unsigned pref = 0u, pmask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int t = threadIdx.x; t < 256; t += NT) h256[t] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += V * NT) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int pos = base + v * NT + (int)threadIdx.x;
        int sc = 0;
        if (pos < n && pred(pos, sc)) {
          const unsigned u = okey(sc);
          if ((u & pmask) == pref) atomicAdd(&h256[(u >> shift) & 255u], 1);
        }
      }
    }
    __syncthreads();
    const int t = threadIdx.x;
    const int c = t < 256 ? h256[255 - t] : 0;
    int tot;
    const int excl = block_exclusive_scan<NT>(c, scan_tmp, &tot);
    if (t < 256 && excl < need && excl + c >= need) {
      sh[0] = 255 - t;
      sh[1] = excl;
    }
    __syncthreads();
    const int d = sh[0];
    need -= sh[1];
    pref |= (unsigned)d << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  *need_eq = need;
  return pref;
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_kernel(const int32_t* __restrict__ scores, long long ld,
                                                  const int32_t* __restrict__ q_pos,
                                                  const int32_t* __restrict__ kept, int bs, int n_keep,
                                                  int L_max, int k, int32_t* __restrict__ idx,
                                                  int32_t* __restrict__ count) {
  constexpr int NW = NT / 64;
  constexpr int VG = 16;  // entries per thread per pass over global memory
  __shared__ int lds_big[NBINS];  // histogram, then the candidate list (slots | scores)
  __shared__ int wcnt[2 * VG * NW];
  __shared__ int scan_tmp[NW + 1];
  __shared__ int h256[256];
  __shared__ int kept_s[256];
  __shared__ int sh[8];

  const long long row = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = min(q_pos[row], L_max - 1);
  const int32_t* srow = scores + row * ld;
  int32_t* out = idx + row * (long long)k;
  const bool is_kept = kept != nullptr;

  int n_slots;
  int n_valid;
  if (is_kept) {
    for (int t = tid; t < n_keep; t += NT) kept_s[t] = kept[row * n_keep + t];
    __syncthreads();
    n_slots = (p >= 0) ? n_keep * bs : 0;
    int c = 0;
    if (tid < n_keep && p >= 0) {
      const int blk = kept_s[tid];
      if (blk >= 0) c = max(0, min(bs, p - blk * bs + 1));
    }
    int tot;
    (void)block_exclusive_scan<NT>(c, scan_tmp, &tot);
    n_valid = tot;
  } else {
    n_slots = max(p + 1, 0);
    n_valid = n_slots;
  }

  auto key_of = [&](int s) -> int {
    if (!is_kept) return s;
    return kept_s[s / bs] * bs + s % bs;
  };
  // candidate test + score load for slot s
  auto cand = [&](int s, int& sc) -> bool {
    if (is_kept) {
      const int blk = kept_s[s / bs];
      if (blk < 0) return false;
      const int j = blk * bs + s % bs;
      if (j > p) return false;
    }
    sc = srow[s];
    return true;
  };

  if (count != nullptr && tid == 0) count[row] = min(k, n_valid);

  // ---- fewer candidates than k: every candidate, in order, then -1 padding
  if (n_valid <= k) {
    ordered_compact<NT, VG>(n_slots, wcnt, [&](int s, int& pl) { int sc; return cand(s, sc); },
                            [&](int r, int s, int) {
                              if (r < k) out[r] = key_of(s);
                            });
    for (int t = n_valid + tid; t < k; t += NT) out[t] = -1;
    return;
  }

  // ---- 1. coarse histogram
  for (int t = tid; t < NBINS; t += NT) lds_big[t] = 0;
  __syncthreads();
  for (int base = 0; base < n_slots; base += VG * NT) {
    int sc[VG];
    bool ok[VG];
#pragma unroll
    for (int v = 0; v < VG; ++v) {
      const int s = base + v * NT + tid;
      sc[v] = 0;
      ok[v] = (s < n_slots) && cand(s, sc[v]);
    }
#pragma unroll
    for (int v = 0; v < VG; ++v)
      if (ok[v]) atomicAdd(&lds_big[coarse_bin(sc[v])], 1);
  }
  __syncthreads();

  // ---- 2. bin holding the k-th best: thread t owns bins [NBINS-(t+1)C, NBINS-tC)
  {
    constexpr int C = NBINS / NT;
    const int hi = NBINS - tid * C;
    int csum = 0;
#pragma unroll 8
    for (int b = hi - C; b < hi; ++b) csum += lds_big[b];
    int tot;
    const int excl = block_exclusive_scan<NT>(csum, scan_tmp, &tot);
    if (excl < k && excl + csum >= k) {
      int acc = excl;
      for (int b = hi - 1; b >= hi - C; --b) {
        const int h = lds_big[b];
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
  const int bstar = sh[4], above = sh[5], cnt_star = sh[6];
  __syncthreads();

  unsigned T;
  int need_eq;
  if (above + cnt_star <= CAP) {
    // ---- 3. list of entries in bins >= b*, in slot order
    int* lslot = lds_big;
    int* lval = lds_big + CAP;
    const int Lc = ordered_compact<NT, VG>(
        n_slots, wcnt,
        [&](int s, int& pl) {
          int sc;
          if (!cand(s, sc)) return false;
          pl = sc;
          return coarse_bin(sc) >= bstar;
        },
        [&](int r, int s, int sc) {
          if (r < CAP) {
            lslot[r] = s;
            lval[r] = sc;
          }
        });
    // ---- 4. exact threshold among the b* entries
    T = radix_select32<NT, 4>(
        Lc, k - above, h256, scan_tmp, sh,
        [&](int e, int& sc) {
          sc = lval[e];
          return coarse_bin(sc) == bstar;
        },
        &need_eq);
    // ---- 5. eq-rank of entries equal to T, then the output compaction
    ordered_compact<NT, 4>(
        Lc, wcnt, [&](int e, int&) { return okey(lval[e]) == T; },
        [&](int r, int e, int) {
          if (r >= need_eq) lslot[e] = -1 - lslot[e];  // mark: equal to T but not taken
        });
    ordered_compact<NT, 4>(
        Lc, wcnt,
        [&](int e, int&) {
          return lslot[e] >= 0 && okey(lval[e]) >= T;
        },
        [&](int r, int e, int) {
          if (r < k) out[r] = key_of(lslot[e]);
        });
  } else {
    // ---- fallback: exact radix passes and compaction over the row in global memory
    T = radix_select32<NT, VG>(n_slots, k, h256, scan_tmp, sh,
                               [&](int s, int& sc) { return cand(s, sc); }, &need_eq);
    // rank among entries equal to T is needed in slot order: count them chunk by chunk
    constexpr int VF = (NBINS / NT < VG) ? NBINS / NT : VG;  // chunk fits lds_big
    int eq_before = 0;
    const int need = need_eq;
    int written = 0;
    for (int base = 0; base < n_slots; base += VF * NT) {
      const int n_here = min(VF * NT, n_slots - base);
      // entries equal to T in this chunk, in order
      int* eq_rank = lds_big;
      const int neq = ordered_compact<NT, VF>(
          n_here, wcnt,
          [&](int e, int&) {
            int sc;
            return cand(base + e, sc) && okey(sc) == T;
          },
          [&](int r, int e, int) { eq_rank[e] = r; });
      const int wr = ordered_compact<NT, VF>(
          n_here, wcnt,
          [&](int e, int&) {
            int sc;
            if (!cand(base + e, sc)) return false;
            const unsigned u = okey(sc);
            return u > T || (u == T && eq_before + eq_rank[e] < need);
          },
          [&](int r, int e, int) {
            if (written + r < k) out[written + r] = key_of(base + e);
          });
      eq_before += neq;
      written += wr;
    }
  }
}

// Block keep of the two-stage indexer: own block + the best n_keep-1 earlier blocks
// by (int64 score desc, block asc), ascending, -1 padded.
template <int NT>
__global__ __launch_bounds__(NT) void blk_select_kernel(const long long* __restrict__ bscores, long long ld,
                                                        const int32_t* __restrict__ q_pos, int n_blocks,
                                                        int bs, int n_keep, int32_t* __restrict__ kept) {
  constexpr int NW = NT / 64;
  constexpr int V = 4;
  __shared__ int wcnt[2 * V * NW];
  __shared__ int scan_tmp[NW + 1];
  __shared__ int h256[256];
  __shared__ unsigned long long shu[4];
  __shared__ int sh[4];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = q_pos[row];
  int32_t* out = kept + row * (long long)n_keep;
  if (p < 0) {
    for (int t = tid; t < n_keep; t += NT) out[t] = -1;
    return;
  }
  const int own = p / bs;
  const int n_sc = min(own, n_blocks);  // scored earlier blocks
  const long long* br = bscores + row * ld;
  auto key64 = [&](int m) -> unsigned long long {
    return (unsigned long long)br[m] ^ 0x8000000000000000ull;
  };
  const int n_sel = min(n_keep - 1, n_sc);
  int written = 0;
  if (n_sel >= n_sc) {
    written = ordered_compact<NT, V>(n_sc, wcnt, [&](int, int&) { return true; },
                                     [&](int r, int m, int) {
                                       if (r < n_keep - 1) out[r] = m;
                                     });
  } else if (n_sel > 0) {
    // max / min of the keys -> bits they all share -> first digit to examine
    unsigned long long mx = 0, mn = ~0ull;
    for (int m = tid; m < n_sc; m += NT) {
      const unsigned long long u = key64(m);
      mx = u > mx ? u : mx;
      mn = u < mn ? u : mn;
    }
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long a = __shfl_xor(mx, o), b = __shfl_xor(mn, o);
      mx = a > mx ? a : mx;
      mn = b < mn ? b : mn;
    }
    if (tid == 0) { shu[0] = 0; shu[1] = ~0ull; }
    __syncthreads();
    if ((tid & 63) == 0) {
      atomicMax(&shu[0], mx);
      atomicMin(&shu[1], mn);
    }
    __syncthreads();
    mx = shu[0];
    mn = shu[1];
    __syncthreads();
    int need = n_sel;
    unsigned long long pref, pmask;
    int shift;
    if (mx == mn) {
      pref = mx;
      pmask = ~0ull;
      shift = -8;
    } else {
      const int hb = 63 - __clzll((long long)(mx ^ mn));  // highest differing bit
      shift = (hb / 8) * 8;
      pmask = (shift + 8 >= 64) ? 0ull : ~((1ull << (shift + 8)) - 1ull);
      pref = mx & pmask;
    }
    for (; shift >= 0; shift -= 8) {
      for (int t = tid; t < 256; t += NT) h256[t] = 0;
      __syncthreads();
      for (int m = tid; m < n_sc; m += NT) {
        const unsigned long long u = key64(m);
        if ((u & pmask) == pref) atomicAdd(&h256[(int)((u >> shift) & 255ull)], 1);
      }
      __syncthreads();
      const int c = tid < 256 ? h256[255 - tid] : 0;
      int tot;
      const int excl = block_exclusive_scan<NT>(c, scan_tmp, &tot);
      if (tid < 256 && excl < need && excl + c >= need) {
        sh[0] = 255 - tid;
        sh[1] = excl;
      }
      __syncthreads();
      need -= sh[1];
      pref |= (unsigned long long)sh[0] << shift;
      pmask |= 255ull << shift;
      __syncthreads();
    }
    const unsigned long long T = pref;
    const int need_eq = need;
    // blocks equal to T beyond the first need_eq are dropped; rank them in order
    __shared__ int drop_from;
    if (tid == 0) drop_from = n_sc;
    __syncthreads();
    ordered_compact<NT, V>(n_sc, wcnt, [&](int m, int&) { return key64(m) == T; },
                           [&](int r, int m, int) {
                             if (r == need_eq) drop_from = m;
                           });
    const int df = drop_from;
    written = ordered_compact<NT, V>(
        n_sc, wcnt,
        [&](int m, int&) {
          const unsigned long long u = key64(m);
          return u > T || (u == T && m < df);
        },
        [&](int r, int m, int) {
          if (r < n_keep - 1) out[r] = m;
        });
  }
  written = min(written, n_keep - 1);
  if (tid == 0) out[written] = own;
  for (int t = written + 1 + tid; t < n_keep; t += NT) out[t] = -1;
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_q;
  if (rows == 0) return hipSuccess;
  if (rows <= 1024 && a.L_max >= 16384) {
    hipLaunchKernelGGL(topk_kernel<1024>, dim3((unsigned)rows), dim3(1024), 0, st, a.scores, a.ld, a.q_pos,
                       a.kept, a.block_size, a.n_keep, a.L_max, a.k, a.idx, a.count);
  } else {
    hipLaunchKernelGGL(topk_kernel<256>, dim3((unsigned)rows), dim3(256), 0, st, a.scores, a.ld, a.q_pos,
                       a.kept, a.block_size, a.n_keep, a.L_max, a.k, a.idx, a.count);
  }
  return hipGetLastError();
}

hipError_t launch_block_select(const BlkSelArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_q;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(blk_select_kernel<256>, dim3((unsigned)rows), dim3(256), 0, st, a.bscores, a.ld,
                     a.q_pos, a.n_blocks, a.block_size, a.n_keep, a.kept);
  return hipGetLastError();
}

}  // namespace lsa
